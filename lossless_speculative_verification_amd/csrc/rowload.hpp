// Row loads shared by every pass over the logits: 16-byte streamed vectors
// (aligned rows) or element gathers (unaligned rows), with -inf past the end.
#pragma once

#include "kernels.hpp"

namespace psi {

// --------------------------------------------------------------- loads --
// Logits are streamed once: 16-byte loads with the nontemporal hint, so that
// they do not displace reusable lines from the caches.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4_t global_u32x4_t;
__device__ __forceinline__ uint4 stream_load(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load((global_u32x4_t*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Loads NV vectors of one row: vector k of this thread is vector index
// vfirst + k * STRIDE (16 bytes each) when aligned, else the same elements one
// by one. Out-of-row elements read as -inf.
template <int DT, bool AL, int NV, int STRIDE>
__device__ __forceinline__ void load_vecs(const char* row, int V, int nvec, int64_t vfirst,
                                          float (&x)[NV][Elem<DT>::kPerVec]) {
  using E = Elem<DT>;
  constexpr int EPV = E::kPerVec;
  if constexpr (AL) {
    const uint4* rp = (const uint4*)row;
    uint4 v[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int64_t idx = vfirst + (int64_t)k * STRIDE;
      v[k] = idx < nvec ? stream_load(rp + idx) : make_uint4(E::kNegInfWord, E::kNegInfWord, E::kNegInfWord, E::kNegInfWord);
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) E::unpack(v[k], x[k]);
  } else {
#pragma unroll
    for (int k = 0; k < NV; ++k)
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const int64_t j = (vfirst + (int64_t)k * STRIDE) * EPV + e;
        x[k][e] = j < V ? E::load1(row, j) : -INFINITY;
      }
  }
}

// Raw 16-byte vectors of one row (same element placement as load_vecs); the
// unaligned path gathers element by element and packs them the same way.
template <int DT, bool AL, int NV, int STRIDE>
__device__ __forceinline__ void load_raw(const char* row, int V, int nvec, int64_t vfirst, uint4 (&v)[NV]) {
  using E = Elem<DT>;
  constexpr int EPV = E::kPerVec;
  if constexpr (AL) {
    const uint4* rp = (const uint4*)row;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int64_t idx = vfirst + (int64_t)k * STRIDE;
      v[k] = idx < nvec ? stream_load(rp + idx) : make_uint4(E::kNegInfWord, E::kNegInfWord, E::kNegInfWord, E::kNegInfWord);
    }
  } else {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (DT == kBF16) {
          const int64_t j0 = (vfirst + (int64_t)k * STRIDE) * EPV + 2 * q;
          const uint32_t lo = j0 < V ? (uint32_t)((const uint16_t*)row)[j0] : 0xff80u;
          const uint32_t hi = j0 + 1 < V ? (uint32_t)((const uint16_t*)row)[j0 + 1] : 0xff80u;
          w[q] = lo | (hi << 16);
        } else {
          const int64_t j = (vfirst + (int64_t)k * STRIDE) * EPV + q;
          w[q] = j < V ? ((const uint32_t*)row)[j] : 0xff800000u;
        }
      }
      v[k] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

template <int N>
__device__ __forceinline__ float pairwise_sum(const float (&e)[N]) {
  if constexpr (N == 8) {
    return ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
  } else {
    return (e[0] + e[1]) + (e[2] + e[3]);
  }
}

__device__ __forceinline__ const char* prow_of(const LinCfg& c, int64_t b, int i) {
  return c.rows.p + ((b * (c.K + 1) + i) * (int64_t)c.V) * c.rows.esz;
}
__device__ __forceinline__ const char* qrow_of(const LinCfg& c, int64_t b, int i) {
  return c.rows.q + ((b * c.K + i) * (int64_t)c.V) * c.rows.esz;
}

}  // namespace psi
