// Device helpers for libpsispec (gfx950, wave64).
//
// Counter-based uniforms: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC'11), with the counter layout the
// public header documents: counter = (draw id, row, request, step),
// key = (lo32 seed, hi32 seed), uniform = first output word / 2^32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace psi {

constexpr int kWG = 256;          // threads per workgroup
constexpr int kWave = 64;         // wave64
constexpr int kWaves = kWG / kWave;
constexpr int kSB = 1024;         // elements per fine-grained sub-block (one wave)
constexpr int kChunk64 = kSB * kWaves;  // elements per workgroup in fp64-grade passes
constexpr uint32_t kDrawFinal = 0u;
constexpr uint32_t kDrawAccept = 1u;
constexpr uint32_t kDrawDraft = 0x40000000u;

// ---------------------------------------------------------------- Philox --
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                 uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = c0 * 0xD2511F53u, hi0 = __umulhi(c0, 0xD2511F53u);
    const uint32_t lo1 = c2 * 0xCD9E8D57u, hi1 = __umulhi(c2, 0xCD9E8D57u);
    const uint32_t n0 = hi1 ^ c1 ^ k0;
    const uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return c0;
}

struct Rng {
  uint32_t k0, k1, step;
  // U(seed, step, b, r, d) in [0, 1) as a double (exact: word * 2^-32).
  __device__ __forceinline__ double u(uint32_t b, uint32_t r, uint32_t d) const {
    return (double)philox_word0(d, r, b, step, k0, k1) * 2.3283064365386962890625e-10;
  }
};

// ------------------------------------------------------------- loading --
// dtype codes of the public header
constexpr int kF32 = 0;
constexpr int kBF16 = 1;

template <int DT>
struct Elem;
template <>
struct Elem<kF32> {
  static constexpr int kBytes = 4;
  static constexpr int kPerVec = 4;  // elements per 16-byte vector
  static constexpr uint32_t kNegInfWord = 0xff800000u;
  __device__ __forceinline__ static void unpack(const uint4& v, float (&x)[4]) {
    x[0] = __uint_as_float(v.x);
    x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z);
    x[3] = __uint_as_float(v.w);
  }
  __device__ __forceinline__ static float load1(const void* base, int64_t idx) {
    return ((const float*)base)[idx];
  }
};
template <>
struct Elem<kBF16> {
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;
  static constexpr uint32_t kNegInfWord = 0xff80ff80u;
  __device__ __forceinline__ static void unpack(const uint4& v, float (&x)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(w[j] << 16);
      x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static float load1(const void* base, int64_t idx) {
    return __uint_as_float((uint32_t)((const uint16_t*)base)[idx] << 16);
  }
};

// NaN-propagating maximum (gfx950 v_maximum3_f32): a NaN anywhere in a row
// makes its maximum NaN, which the statistics then carry to the row verdict.
__device__ __forceinline__ float fmaxnan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ bool is_neg_inf(float x) { return __float_as_uint(x) == 0xff800000u; }
__device__ __forceinline__ bool is_neg_inf(double x) {
  return __double_as_longlong(x) == (long long)0xfff0000000000000ull;
}

// --------------------------------------------------------- reductions --
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxnan(v, __shfl_xor(v, o));
  return v;
}
// fp64 lane moves inside the VALU (DPP), for scans and sums without LDS
// permutes: CTRL is a DPP control (row_shr:n = 0x110 + n, row_bcast:15 =
// 0x142, row_bcast:31 = 0x143), ROWS the rows of 16 lanes that receive; lanes
// that receive nothing read 0.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROWS, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROWS, 0xf, true);
  return __hiloint2double(hi, lo);
}

// Inclusive sum over the lanes of a wave, in lane order: within each row of
// 16 by shifts of 1, 2, 4, 8, then across rows by broadcasting lane 15 of
// rows 0 and 2 and lane 31 (Hillis-Steele on DPP).
__device__ __forceinline__ double wave_incl_scan(double v) {
  v += dpp_f64<0x111, 0xf>(v);
  v += dpp_f64<0x112, 0xf>(v);
  v += dpp_f64<0x114, 0xf>(v);
  v += dpp_f64<0x118, 0xf>(v);
  v += dpp_f64<0x142, 0xa>(v);
  v += dpp_f64<0x143, 0xc>(v);
  return v;
}

// Sum over the wave, the same on every lane, by the DPP scan (lane 63 of the
// inclusive sum, read back): VALU lane moves instead of LDS permutes, for
// latency-bound paths with few waves per SIMD. The order of the additions is
// the scan's.
__device__ __forceinline__ double wave_sum_dpp(double v) {
  v = wave_incl_scan(v);
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), kWave - 1);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), kWave - 1);
  return __hiloint2double(hi, lo);
}

// Sum over the wave, the same on every lane (butterfly).
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// Sums of four values over the wave with one butterfly: after exchanging
// halves at lane distance 32 and 16, each 16-lane group holds partial sums of
// one value and finishes it alone. Lanes 0-15 end with sum(v0), 16-31 with
// sum(v1), 32-47 with sum(v2), 48-63 with sum(v3). 14 lane permutes instead
// of 48 for four separate reductions.
__device__ __forceinline__ double wave_sum4(double v0, double v1, double v2, double v3) {
  const int lane = threadIdx.x & (kWave - 1);
  const bool hi32 = lane & 32, hi16 = lane & 16;
  const double r0 = __shfl_xor(hi32 ? v0 : v2, 32), r1 = __shfl_xor(hi32 ? v1 : v3, 32);
  const double k0 = (hi32 ? v2 : v0) + r0, k1 = (hi32 ? v3 : v1) + r1;
  double k = (hi16 ? k1 : k0) + __shfl_xor(hi16 ? k0 : k1, 16);
  k += __shfl_xor(k, 8);
  k += __shfl_xor(k, 4);
  k += __shfl_xor(k, 2);
  k += __shfl_xor(k, 1);
  return k;
}

// Orders the LDS accesses of one wave around this point (the wave's LDS
// operations complete in issue order; this keeps the compiler from moving
// them across it).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Maximum of an unsigned value over the wave, on every lane: within rows of 16
// by shifts of 1, 2, 4, 8, across rows by the row broadcasts (as in
// wave_incl_scan), then lane 63 is read.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, true));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v |= __shfl_xor(v, o);
  return v;
}

// Workgroup-wide reductions over NT threads in a fixed order (deterministic);
// `sh` needs NT / kWave slots.
template <int NT = kWG>
__device__ __forceinline__ float block_max(float v, float* sh) {
  constexpr int NW = NT / kWave;
  v = wave_max(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = fmaxnan(r, sh[i]);
  return r;
}
template <int NT = kWG>
__device__ __forceinline__ double block_sum(double v, double* sh) {
  constexpr int NW = NT / kWave;
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh[w] = v;
  __syncthreads();
  double r = sh[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r += sh[i];
  return r;
}

// Exclusive scan of one double per thread across NT threads, in thread order;
// returns the exclusive prefix and writes the total. `sh` needs NT + NT / kWave
// slots. Each wave scans in registers, then the wave totals are scanned.
template <int NT = kWG>
__device__ __forceinline__ double block_exclusive_scan(double v, double* sh, double* total) {
  constexpr int NW = NT / kWave;
  const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
  const double incl = wave_incl_scan(v);
  __syncthreads();
  if (lane == kWave - 1) sh[w] = incl;
  __syncthreads();
  double before = 0.0, all = 0.0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const double x = sh[i];
    if (i < w) before += x;
    all += x;
  }
  *total = all;
  __syncthreads();
  return before + (incl - v);
}

// 2^y in fp64 for y <= 1023 (relative error < 5e-16; 0 for y below -1022,
// -inf and NaN included). k = the integer nearest y is
// read from the low word of y + 1.5 * 2^52, f = y - k lies in [-1/2, 1/2],
// 2^f comes from a degree-10 near-minimax polynomial (Chebyshev interpolation
// at 11 nodes, coefficients from exp2_coeffs.py), and 2^k is assembled in the
// exponent field. Only full-rate fp64 and integer operations.
__device__ __forceinline__ double exp2_fast(double y0) {
  const double y = fmax(y0, -1022.0);
  constexpr double kMagic = 6755399441055744.0;  // 1.5 * 2^52
  const double t = y + kMagic;
  const double f = y - (t - kMagic);
  const int k = __double2loint(t);
  double p = 7.072587226569927e-09;
  p = __builtin_fma(p, f, 1.0208690586037056e-07);
  p = __builtin_fma(p, f, 1.3215442576793237e-06);
  p = __builtin_fma(p, f, 1.5252657258547322e-05);
  p = __builtin_fma(p, f, 0.00015403530441763784);
  p = __builtin_fma(p, f, 0.001333355823016814);
  p = __builtin_fma(p, f, 0.00961812910760687);
  p = __builtin_fma(p, f, 0.055504108664447695);
  p = __builtin_fma(p, f, 0.24022650695910097);
  p = __builtin_fma(p, f, 0.69314718055995);
  p = __builtin_fma(p, f, 1.0);
  const double r = p * __hiloint2double((k + 1023) << 20, 0);
  return y0 >= -1022.0 ? r : 0.0;
}

}  // namespace psi
