// NVFP4 quantiser on gfx950: a bf16 / fp16 / fp32 matrix -> E2M1 codes and
// UE4M3 block scales in the 128x4 layout -- the producer of the operands that
// flashinfer.gemm.mm_nvfp4_lora consumes (the paragraph after its formula:
// the layout fp4_quantize() writes; its alpha parameter: a per-tensor global
// scale g on each operand).
//
// For each row and each block of 16 consecutive elements x_i along K (every
// step an IEEE fp32 operation, round to nearest even):
//   amax = max |x_i|;  s = (amax * g) / 6;  sf = UE4M3(s) nearest, ties to the
//   even code, saturating at 448;  S = value(sf);  r = g / S (0 if S == 0);
//   code_i = E2M1(x_i * r) nearest, ties to the even code, saturating at 6,
//   sign bit from the sign of the product.
// The scale rounding is integer logic on the fp32 bit pattern; the element
// rounding is v_cvt_scalef32_pk_fp4_f32 at scale 1.0, which rounds to the
// nearest E2M1 value with ties to the even code, saturates at 6 and keeps the
// sign -- the definition (checked bitwise against the oracle, midpoints and
// saturation included, by the GPU tests).
//
// Work split: HBM-bound.  Lane j of a wavefront holds 8 consecutive elements
// (one 16-byte load for 16-bit inputs), so each load instruction of a
// wavefront reads 1 KiB contiguous; lanes 2m and 2m+1 form a 16-element block
// (amax through one lane swap), lanes 8q .. 8q+7 the 4 blocks of one 4-byte
// scale word, which lane 8q writes.  Each lane writes its 8 codes as one
// 32-bit word (coalesced).  K % 64 == 0 keeps every scale word inside a row.
#include "common.hpp"

namespace mi {
namespace {

constexpr int QZ_THREADS = 256;
constexpr int QZ_SEG = 4;  // 64-chunk segments per wavefront (loads in flight per lane)

// fp32 v >= 0 (or +inf) -> UE4M3 code: nearest, ties to even, saturating at 0x7E (448)
__device__ __forceinline__ uint32_t ue4m3_rne_sat(float v) {
  if (!(v < 448.f)) return 0x7Eu;
  if (v < 0.015625f)  // below 2^-6: subnormal codes M * 2^-9 (code 8 is 2^-6, the first normal)
    return static_cast<uint32_t>(__builtin_rintf(v * 512.f));
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFFu + ((u >> 20) & 1u);  // round the mantissa to 3 bits, ties to even
  const uint32_t e = (u >> 23) - 127u + 7u;  // E4M3 biased exponent, 1 .. 15
  return min((e << 3) | ((u >> 20) & 7u), 0x7Eu);
}

// UE4M3 code -> its value (exact)
__device__ __forceinline__ float ue4m3_value(uint32_t c) {
  const int E = static_cast<int>(c >> 3), M = static_cast<int>(c & 7u);
  return E == 0 ? __builtin_amdgcn_ldexpf(static_cast<float>(M), -9)
                : __builtin_amdgcn_ldexpf(static_cast<float>(8 + M), E - 10);
}


template <typename T>
struct Chunk8;  // 8 consecutive input elements of one lane
template <>
struct Chunk8<uint16_t> {  // bf16
  u32x4 v;
  __device__ void load(const uint16_t* p) { v = gld_nt<u32x4>(p); }
  __device__ float at(int i) const {
    const uint32_t w = v[i >> 1];
    return __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
};
template <>
struct Chunk8<_Float16> {
  u32x4 v;
  __device__ void load(const _Float16* p) { v = gld_nt<u32x4>(p); }
  __device__ float at(int i) const {
    const uint32_t w = v[i >> 1];
    const uint16_t h = static_cast<uint16_t>((i & 1) ? (w >> 16) : (w & 0xFFFFu));
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
  }
};
template <>
struct Chunk8<float> {
  f32x4 a, b;
  __device__ void load(const float* p) {
    a = gld_nt<f32x4>(p);
    b = gld_nt<f32x4>(p + 4);
  }
  __device__ float at(int i) const { return i < 4 ? a[i] : b[i - 4]; }
};

struct QzArgs {
  const void* x;
  const float* gscale;  // [batch]
  uint8_t* codes;       // [batch, rows, k/2]
  uint8_t* sf;          // batch consecutive 128x4 buffers of sf_per bytes
  long chunks;          // batch * rows * k / 8
  uint32_t per_batch;   // rows * k / 8 chunks of one matrix (< 2^31)
  uint32_t cpr;         // chunks per row (k / 8)
  int nct;              // 128x4 tiles along K (k / 64)
  int batched;          // batch > 1
  long sf_per;
};

__device__ __forceinline__ long sf_word_off(int row, int ct, int nct) {
  return (static_cast<long>(row >> 7) * nct + ct) * 512 + (row & 31) * 16 + ((row & 127) >> 5) * 4;
}

// the quantiser's loads and arithmetic for one wavefront; TAB: r comes from
// the workgroup's table s_r (its chunks all lie in matrix b0 of the batch)
template <typename T, bool TAB>
__device__ __forceinline__ void qz_wave(const QzArgs& p, const float* s_r, uint32_t b0) {
  const int lane = threadIdx.x & 63;
  const long wave = (static_cast<long>(blockIdx.x) * QZ_THREADS + threadIdx.x) >> 6;
  const T* x = static_cast<const T*>(p.x);
  const float g0 = TAB ? gld<float>(p.gscale + b0) : 0.f;
  Chunk8<T> ch[QZ_SEG];
  long c[QZ_SEG];
#pragma unroll
  for (int j = 0; j < QZ_SEG; ++j) {  // every load of the lane first
    c[j] = (wave * QZ_SEG + j) * 64 + lane;
    if (c[j] < p.chunks) ch[j].load(x + c[j] * 8);
  }
#pragma unroll
  for (int j = 0; j < QZ_SEG; ++j) {
    // the whole wavefront reaches the shuffles; chunks past the end compute
    // on whatever their registers hold and store nothing
    const bool in = c[j] < p.chunks;
    const uint32_t bi =
        TAB ? b0 : ((in && p.batched) ? static_cast<uint32_t>(c[j] / p.per_batch) : 0u);
    const float g = TAB ? g0 : (in ? gld<float>(p.gscale + bi) : 0.f);
    float xs[8], am = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      xs[i] = ch[j].at(i);
      am = fmaxf(am, fabsf(xs[i]));
    }
    am = fmaxf(am, __shfl_xor(am, 1));  // the block's other 8 elements
    const uint32_t sfc = ue4m3_rne_sat(__fdiv_rn(__fmul_rn(am, g), 6.f));
    float r;
    if constexpr (TAB) {
      r = s_r[sfc];
    } else {
      const float S = ue4m3_value(sfc);
      r = S == 0.f ? 0.f : __fdiv_rn(g, S);
    }
    // the 8 codes, element 2i in the low nibble of byte i
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __fmul_rn(xs[0], r), __fmul_rn(xs[1], r),
                                                 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __fmul_rn(xs[2], r), __fmul_rn(xs[3], r),
                                                 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __fmul_rn(xs[4], r), __fmul_rn(xs[5], r),
                                                 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __fmul_rn(xs[6], r), __fmul_rn(xs[7], r),
                                                 1.0f, 3);
    // scale word of lanes 8q .. 8q+7: the blocks of lanes 8q, 8q+2, 8q+4, 8q+6
    const int b8 = lane & ~7;
    const uint32_t sw = static_cast<uint32_t>(__shfl(static_cast<int>(sfc), b8)) |
                        static_cast<uint32_t>(__shfl(static_cast<int>(sfc), b8 + 2)) << 8 |
                        static_cast<uint32_t>(__shfl(static_cast<int>(sfc), b8 + 4)) << 16 |
                        static_cast<uint32_t>(__shfl(static_cast<int>(sfc), b8 + 6)) << 24;
    if (!in) continue;
    gst<uint32_t>(p.codes + c[j] * 4, w);
    if ((lane & 7) == 0) {
      // chunk index inside the matrix -> row and 64-element column group
      const uint32_t cm = static_cast<uint32_t>(c[j] - static_cast<long>(bi) * p.per_batch);
      const uint32_t row = cm / p.cpr, cg = (cm - row * p.cpr) >> 3;
      gst<uint32_t>(p.sf + bi * p.sf_per + sf_word_off(static_cast<int>(row), cg, p.nct), sw);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(QZ_THREADS) void fp4_quantize_kernel(QzArgs p) {
  // r = g / S for every UE4M3 code, when the workgroup's chunks all lie in one
  // matrix of the batch (always for batch 1): the same fp32 division per
  // code, once per workgroup instead of once per block.  Built before any
  // input load is issued, so the barrier waits for nothing in flight.
  __shared__ float s_r[128];
  constexpr long WGC = (QZ_THREADS / 64) * QZ_SEG * 64;  // chunks of a workgroup
  const long w0 = static_cast<long>(blockIdx.x) * WGC;
  const long w1 = min(w0 + WGC, p.chunks) - 1;
  const uint32_t b0 = p.batched ? static_cast<uint32_t>(w0 / p.per_batch) : 0u;
  const bool one = !p.batched || static_cast<uint32_t>(w1 / p.per_batch) == b0;
  if (one) {
    if (threadIdx.x < 128) {
      const float g = gld<float>(p.gscale + b0);
      const float S = ue4m3_value(threadIdx.x);
      s_r[threadIdx.x] = S == 0.f ? 0.f : __fdiv_rn(g, S);
    }
    __syncthreads();
    qz_wave<T, true>(p, s_r, b0);
  } else {
    qz_wave<T, false>(p, s_r, 0u);
  }
}

// zero scale words of the padding rows [rows, rows rounded up to 128) of
// every matrix of the batch
__global__ void fp4_sf_pad_kernel(uint8_t* sf, long sf_per, int rows, int pad_rows, int nct,
                                  long total) {
  const long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const long per = static_cast<long>(pad_rows) * nct;  // padding words per matrix
  const long bi = i / per, w = i % per;
  const int row = rows + static_cast<int>(w / nct), ct = static_cast<int>(w % nct);
  gst<uint32_t>(sf + bi * sf_per + sf_word_off(row, ct, nct), 0u);
}

size_t qz_sf_bytes(int64_t rows, int64_t k) {
  return static_cast<size_t>((rows + 127) / 128) * static_cast<size_t>(k / 64) * 512;
}

}  // namespace
}  // namespace mi

extern "C" mi_status mi_fp4_quantize(const void* x, int64_t batch, int64_t rows, int64_t k,
                                     mi_dtype x_dtype, const float* global_scale, uint8_t* codes,
                                     uint8_t* sf, size_t sf_bytes, void* stream) {
  using namespace mi;
  clear_error();
  MI_REQUIRE(batch >= 1, "fp4_quantize: batch must be >= 1 (got %lld)", (long long)batch);
  MI_REQUIRE(rows >= 0 && rows < (1LL << 31), "fp4_quantize: rows out of range");
  MI_REQUIRE(k >= 64 && k % 64 == 0 && k < (1LL << 31),
             "fp4_quantize: K must be a positive multiple of 64 (got %lld)", (long long)k);
  MI_REQUIRE(x_dtype == MI_BF16 || x_dtype == MI_F16 || x_dtype == MI_F32,
             "fp4_quantize: x must be bf16, fp16 or fp32");
  const size_t per = qz_sf_bytes(rows, k);
  MI_REQUIRE(batch * rows * k < (1LL << 40) && per * static_cast<size_t>(batch) < (1ULL << 40) &&
                 rows * (k / 8) < (1LL << 31),
             "fp4_quantize: problem too large");
  if (rows == 0) return MI_OK;
  MI_REQUIRE(x && global_scale && codes && sf, "fp4_quantize: null pointer argument");
  MI_REQUIRE(sf_bytes >= per * static_cast<size_t>(batch),
             "fp4_quantize: sf holds %zu bytes, %lld 128x4 layouts of %lld x %lld need %zu",
             sf_bytes, (long long)batch, (long long)rows, (long long)k,
             per * static_cast<size_t>(batch));
  MI_REQUIRE(aligned16(x) && (reinterpret_cast<uintptr_t>(codes) & 3) == 0 &&
                 (reinterpret_cast<uintptr_t>(sf) & 3) == 0,
             "fp4_quantize: x must be 16-byte aligned, codes and sf 4-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  QzArgs a;
  a.x = x;
  a.gscale = global_scale;
  a.codes = codes;
  a.sf = sf;
  a.per_batch = static_cast<uint32_t>(rows * k / 8);
  a.chunks = batch * static_cast<long>(a.per_batch);
  a.cpr = static_cast<uint32_t>(k / 8);
  a.batched = batch > 1;
  a.nct = static_cast<int>(k / 64);
  a.sf_per = static_cast<long>(per);
  const long waves = (a.chunks + 64 * QZ_SEG - 1) / (64 * QZ_SEG);
  const long grid = (waves + QZ_THREADS / 64 - 1) / (QZ_THREADS / 64);
  MI_REQUIRE(grid < (1L << 31), "fp4_quantize: problem too large");
  switch (x_dtype) {
    case MI_BF16:
      hipLaunchKernelGGL(fp4_quantize_kernel<uint16_t>, dim3(grid), dim3(QZ_THREADS), 0, s, a);
      break;
    case MI_F16:
      hipLaunchKernelGGL(fp4_quantize_kernel<_Float16>, dim3(grid), dim3(QZ_THREADS), 0, s, a);
      break;
    default:
      hipLaunchKernelGGL(fp4_quantize_kernel<float>, dim3(grid), dim3(QZ_THREADS), 0, s, a);
      break;
  }
  mi_status st = launch_status("fp4_quantize");
  if (st != MI_OK) return st;
  const int pad_rows = static_cast<int>((rows + 127) / 128 * 128 - rows);
  if (pad_rows > 0) {
    const long total = batch * pad_rows * (k / 64);
    hipLaunchKernelGGL(fp4_sf_pad_kernel, dim3((total + 255) / 256), dim3(256), 0, s, sf,
                       static_cast<long>(per), static_cast<int>(rows), pad_rows,
                       static_cast<int>(k / 64), total);
    st = launch_status("fp4_quantize (scale padding)");
  }
  return st;
}
