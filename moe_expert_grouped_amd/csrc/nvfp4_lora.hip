// NVFP4 GEMM with a BF16 LoRA epilogue, the prepared-path fold, and the
// NVFP4 dequantiser -- gfx950.
//
// What is computed (flashinfer.gemm.mm_nvfp4_lora, formula and the raw /
// prepared bullets; flashinfer.gemm.prepare_nvfp4_lora_adapter, the fold):
//   raw      out = bf16( alpha*acc + lora_scale*(d @ lora_b^T) [+ bias] )
//   prepared out = bf16( alpha*(acc + d @ b_folded^T) [+ bias] )
//   off      out = bf16( alpha*acc [+ bias] )
// with acc = dequant(a) @ dequant(b)^T in fp32 and one final rounding.
//
// Decoding.  An E2M1 value (<= 2 significant bits) times a UE4M3 scale
// (<= 4 significant bits, 2^-9 .. 448) has at most 6 significant bits and
// lies in 2^-10 .. 2688, so it is exact in fp16.  Each byte of codes becomes
// an fp16 pair with v_cvt_scalef32_pk_f16_fp4 at scale 1.0 (a pure format
// conversion, exact), and one v_pk_mul_f16 by the block's scale (converted
// exactly from its E4M3 byte) applies the scale -- exact as well.  Each lane
// decodes its own MFMA operands in registers (no LDS) and feeds
// v_mfma_f32_32x32x16_f16.  CDNA4's block-scaled MFMA takes power-of-two
// (E8M0) scales on 32-wide blocks, so it cannot consume UE4M3 scales on
// 16-wide blocks; this decode-to-fp16 route is exact instead.
//
// The LoRA term is an epilogue: after the K loop each 32x32 block gets one
// bf16 MFMA per 16 ranks -- into the base accumulator on the prepared path,
// into a separate fp32 accumulator on the raw path.  The adapter-off, raw
// scale-0 and prepared zero-adapter cases all take the same epilogue code
// with the LoRA skipped (the scale / the fold's zero flag is read on the
// device), so their outputs are bitwise identical.  Epilogue arithmetic uses
// explicitly rounded fp32 operations (no contraction).
#include "common.hpp"

namespace mi {
namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int NV_BM = 256, NV_BN = 256;  // workgroup tile
constexpr int NV_KC = 128;               // K elements per register stage (64 code bytes)
constexpr int NV_WM = 2, NV_WN = 2;      // 4 wavefronts of 128 x 128
constexpr int NV_NT = 64 * NV_WM * NV_WN;
constexpr int NV_GROUP_M = 4;

// Byte offset of the UE4M3 scale of (row, scale column col) in the 128x4
// tiled layout: 512-byte tiles of 128 rows x 4 columns, row-block major;
// inside a tile (row%32)*16 + ((row%128)/32)*4 + col%4.  n_col_tiles =
// ceil(k/16/4).  Columns col..col+3 with col%4 == 0 are 4 consecutive bytes.
__device__ __forceinline__ long sf_tile_word(int row, int col4, int n_col_tiles) {
  return (static_cast<long>(row >> 7) * n_col_tiles + col4) * 512 + (row & 31) * 16 +
         ((row & 127) >> 5) * 4;
}

// The scale decode shared by the GEMM K loops and the dequantiser: the four
// UE4M3 bytes of one 32-bit scale word (scale columns 4c .. 4c+3 of a row) as
// fp16, two bytes per conversion -- s01 = (byte 0, byte 1), s23 = (byte 2,
// byte 3).  Exact: a UE4M3 value has at most 4 significant bits and lies in
// 2^-9 .. 448, inside fp16's normal range.
__device__ __forceinline__ void ue4m3x4_to_f16(uint32_t w, f16x2& s01, f16x2& s23) {
  s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
}

// Scale byte c (0..3) of the word as an fp16 pair (s, s): the multiplier of
// decode8 below.
__device__ __forceinline__ f16x2 scale_splat(f16x2 s01, f16x2 s23, int c) {
  const f16x2 v = c < 2 ? s01 : s23;
  return (c & 1) ? f16x2{v.y, v.y} : f16x2{v.x, v.x};
}

// 8 E2M1 codes (one 32-bit word, element 2i in the low nibble of byte i)
// times an fp16 scale pair -> 8 fp16 values, element order preserved.
__device__ __forceinline__ u32x4 decode8(uint32_t w, f16x2 s) {
  u32x4 r;
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  r.x = __builtin_bit_cast(uint32_t, p0);
  r.y = __builtin_bit_cast(uint32_t, p1);
  r.z = __builtin_bit_cast(uint32_t, p2);
  r.w = __builtin_bit_cast(uint32_t, p3);
  return r;
}

__device__ __forceinline__ uint32_t f16_to_bf16_bits(uint32_t h) {
  // exact: every decoded value is representable in bf16
  const float f = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
  return __float_as_uint(f) >> 16;
}

// ---------------------------------------------------------------------------
// NVFP4 GEMM + LoRA epilogue
// ---------------------------------------------------------------------------
struct NvArgs {
  const uint8_t* a;
  const uint8_t* b;
  const uint8_t* a_sf;
  const uint8_t* b_sf;
  const float* alpha;
  const uint16_t* d;
  const uint16_t* lora_b;    // raw path
  const float* lora_scale;   // raw path (NULL -> off)
  const uint16_t* b_folded;  // prepared path
  const uint32_t* fold_flags;
  const uint16_t* bias;
  uint16_t* out;
  int m, n, k, rank;
  int mode;  // 0 off, 1 raw, 2 prepared
};

// One register stage of a wavefront: for each of its 4 A and 4 B fragment
// rows, this lane's 64 codes (32 bytes) and their 4 scale bytes.
struct NvStage {
  u32x4 a[4][2], b[4][2];
  uint32_t sa[4], sb[4];
};

// Operands of one wavefront's 128 x 128 block: buffer descriptors of codes
// and scales, and the lane's byte offsets of its 4 A and 4 B fragment rows
// (codes: the row's first byte plus 32 * lane half; scales: its 128x4 word).
struct NvOps {
  __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
  uint32_t oa[4], ob[4], osa[4], osb[4];
};

// The K loop of one wavefront (NKC stages of 128, NKC even): acc = dequant(A
// rows) x dequant(B rows)^T in fp32.  B is the MFMA's first operand, so
// acc[i][j][q] is A row 32 i + lane % 32 and B row 32 j + 8 (q / 4) +
// 4 (lane / 32) + q % 4: four consecutive output columns per lane and q / 4.
__device__ __forceinline__ void nv_kloop(f32x16 (&acc)[4][4], const NvOps& op, int NKC) {
  constexpr int FM = 4, FN = 4;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  // stage kc: codes at byte kc*64 of the row, scales in scale tile 2*kc + h
  auto load = [&](NvStage& st, int kc) {
    const uint32_t co = static_cast<uint32_t>(kc) * (NV_KC / 2);
    const uint32_t so = static_cast<uint32_t>(kc) * 1024;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      st.a[i][0] = buf_ld128(op.ra, op.oa[i], co);
      st.a[i][1] = buf_ld128(op.ra, op.oa[i] + 16, co);
      st.sa[i] = buf_ld32(op.rsa, op.osa[i], so);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      st.b[j][0] = buf_ld128(op.rb, op.ob[j], co);
      st.b[j][1] = buf_ld128(op.rb, op.ob[j] + 16, co);
      st.sb[j] = buf_ld32(op.rsb, op.osb[j], so);
    }
  };
  auto compute = [&](const NvStage& st) {
    // the 4 UE4M3 scale bytes of each row as fp16, two per conversion (exact)
    f16x2 sa01[FM], sa23[FM], sb01[FN], sb23[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) ue4m3x4_to_f16(st.sa[i], sa01[i], sa23[i]);
#pragma unroll
    for (int j = 0; j < FN; ++j) ue4m3x4_to_f16(st.sb[j], sb01[j], sb23[j]);
#pragma unroll
    for (int t = 0; t < 4; ++t) {  // scale block t: MFMA steps 2t, 2t+1
      f16x2 psa[FM], psb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) psa[i] = scale_splat(sa01[i], sa23[i], t);
#pragma unroll
      for (int j = 0; j < FN; ++j) psb[j] = scale_splat(sb01[j], sb23[j], t);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int s = 2 * t + u;  // code word s of the lane's 8
        u32x4 fa[FM], fb[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[i] = decode8(st.a[i][s >> 2][s & 3], psa[i]);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[j] = decode8(st.b[j][s >> 2][s & 3], psb[j]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(f16x8, fb[j]), __builtin_bit_cast(f16x8, fa[i]), acc[i][j], 0,
                0, 0);
      }
    }
    // interleave: the decode of later steps runs while earlier MFMAs execute
#pragma unroll
    for (int g = 0; g < 8 * FM * FN; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // five VALU
    }
  };

  // K / 128 is even (K % 256 == 0): two stages per trip, the refill index is
  // clamped so every trip issues the same loads
  NvStage s0, s1;
  load(s0, 0);
  for (int kc = 0; kc < NKC; kc += 2) {
    // the barriers keep each refill where it is issued: a whole stage ahead
    load(s1, kc + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(s0);
    __builtin_amdgcn_sched_barrier(0);
    load(s0, min(kc + 2, NKC - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(s1);
    __builtin_amdgcn_sched_barrier(0);
  }

}

// One wavefront computes a 128 x 128 block as 4 x 4 v_mfma_f32_32x32x16_f16
// tiles; the accumulators (256 floats a lane) live in AGPRs.  There is no LDS:
// the sum over K is order-free, so inside every 128-wide K stage lane half h
// (lane / 32) takes the 64 consecutive elements [64h, 64h + 64) and MFMA step
// s (0..7) consumes elements 64h + 8s .. +7 from both halves -- A and B use
// the same assignment.  Each lane therefore reads its row's codes as 32
// contiguous bytes and decodes them straight into MFMA operands.  Every A and
// B row is decoded by the two wavefronts that share it.
__global__ __launch_bounds__(NV_NT, 1) void nvfp4_lora_kernel(NvArgs p) {
  constexpr int WTM = NV_BM / NV_WM, WTN = NV_BN / NV_WN;  // 128 x 128
  constexpr int FM = WTM / 32, FN = WTN / 32;               // 4 x 4

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NV_WN, wn = wave % NV_WN;

  // ---- tile order: XCD-contiguous runs, GROUP_M m-tiles per n sweep ----
  const int mt = (p.m + NV_BM - 1) / NV_BM, ntile = (p.n + NV_BN - 1) / NV_BN;
  const int total = mt * ntile;
  const int G = gridDim.x;  // == total rounded up to a multiple of 8
  const int L = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  if (L >= total) return;
  const int span = NV_GROUP_M * ntile;
  const int grp = L / span, first = grp * NV_GROUP_M;
  const int gsize = min(mt - first, NV_GROUP_M);
  const int in_grp = L - grp * span;
  const int m0 = (first + in_grp % gsize) * NV_BM;
  const int n0 = (in_grp / gsize) * NV_BN;

  // ---- per-lane byte offsets (codes and scales), rows clamped into range ----
  const int r32 = lane & 31, h = lane >> 5;
  const uint32_t kb = static_cast<uint32_t>(p.k) / 2;  // code bytes per row
  const int nct = (p.k / 16 + 3) / 4;                   // 128x4 scale tiles along K
  NvOps op;
  op.ra = buf_rsrc(p.a, static_cast<uint32_t>(p.m) * kb);
  op.rb = buf_rsrc(p.b, static_cast<uint32_t>(p.n) * kb);
  op.rsa = buf_rsrc(p.a_sf, static_cast<uint32_t>((p.m + 127) / 128) * nct * 512);
  op.rsb = buf_rsrc(p.b_sf, static_cast<uint32_t>((p.n + 127) / 128) * nct * 512);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int row = min(m0 + wm * WTM + i * 32 + r32, p.m - 1);
    op.oa[i] = static_cast<uint32_t>(row) * kb + h * 32;
    op.osa[i] = static_cast<uint32_t>(sf_tile_word(row, h, nct));
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int row = min(n0 + wn * WTN + j * 32 + r32, p.n - 1);
    op.ob[j] = static_cast<uint32_t>(row) * kb + h * 32;
    op.osb[j] = static_cast<uint32_t>(sf_tile_word(row, h, nct));
  }

  f32x16 acc[FM][FN];
  nv_kloop(acc, op, p.k / NV_KC);

  // ---- epilogue ----
  const float alpha = p.alpha[0];
  bool lora = false;
  float s_lora = 0.f;
  const uint16_t* lb = nullptr;
  if (p.mode == 1) {
    s_lora = p.lora_scale[0];
    lora = (s_lora != 0.f);
    lb = p.lora_b;
  } else if (p.mode == 2) {
    lora = (p.fold_flags[0] & 1u) == 0u;
    lb = p.b_folded;
  }
  const int kl = lane >> 5;  // which 8-rank half of a 16-rank step this lane feeds
  // 4 consecutive bf16 columns per 8-byte store where the rows allow it
  const bool vec = (p.n & 3) == 0 && (reinterpret_cast<uintptr_t>(p.out) & 7) == 0;
  const bool has_bias = p.bias != nullptr;
  const bool raw_lora = lora && p.mode == 1;

#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int cbase = n0 + wn * WTN + j * 32;
    // the lane's columns cbase + 8 g + 4 kl + c: bias values (zero past the end)
    float bv[4][4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int col = cbase + 8 * g + 4 * kl + c;
        bv[g][c] = (has_bias && col < p.n) ? bf16_bits_to_f32(p.bias[col]) : 0.f;
      }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int rbase = m0 + wm * WTM + i * 32;
      f32x16 accl;
#pragma unroll
      for (int q = 0; q < 16; ++q) accl[q] = 0.f;
      if (lora) {
        // d rows rbase..+31 (clamped), lb rows cbase..+31 (clamped); K = rank; lb
        // is the first operand, as in the K loop
        const int dr = min(rbase + (lane & 31), p.m - 1);
        const int br = min(cbase + (lane & 31), p.n - 1);
        const uint16_t* dp = p.d + static_cast<long>(dr) * p.rank + kl * 8;
        const uint16_t* bp = lb + static_cast<long>(br) * p.rank + kl * 8;
        if (p.mode == 2) {
          for (int r0 = 0; r0 < p.rank; r0 += 16) {
            u32x4 fd = {0, 0, 0, 0}, fl = {0, 0, 0, 0};
            if (r0 + kl * 8 < p.rank) {
              fd = *reinterpret_cast<const u32x4*>(dp + r0);
              fl = *reinterpret_cast<const u32x4*>(bp + r0);
            }
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, fl), __builtin_bit_cast(bf16x8, fd), acc[i][j], 0, 0, 0);
          }
        } else {
          for (int r0 = 0; r0 < p.rank; r0 += 16) {
            u32x4 fd = {0, 0, 0, 0}, fl = {0, 0, 0, 0};
            if (r0 + kl * 8 < p.rank) {
              fd = *reinterpret_cast<const u32x4*>(dp + r0);
              fl = *reinterpret_cast<const u32x4*>(bp + r0);
            }
            accl = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, fl), __builtin_bit_cast(bf16x8, fd), accl, 0, 0, 0);
          }
        }
      }
      const int row = rbase + (lane & 31);
      if (row < p.m) {
        uint16_t* orow = p.out + static_cast<long>(row) * p.n;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c0 = cbase + 8 * g + 4 * kl;
          uint32_t w[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int q = 4 * g + c;
            float v = __fmul_rn(alpha, acc[i][j][q]);
            if (raw_lora) v = __fadd_rn(v, __fmul_rn(s_lora, accl[q]));
            if (has_bias) v = __fadd_rn(v, bv[g][c]);
            w[c] = f32_to_bf16_rne(v);
          }
          if (vec) {
            if (c0 < p.n)  // n % 4 == 0: all four columns are in range
              *reinterpret_cast<u32x2*>(orow + c0) = u32x2{w[0] | (w[1] << 16), w[2] | (w[3] << 16)};
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (c0 + c < p.n) orow[c0 + c] = static_cast<uint16_t>(w[c]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// NVFP4 grouped GEMM: the ragged per-expert walk with FP4 expert weights
//   out[m_indptr[e]:m_indptr[e+1]] = alpha[e] * dequant(a[...]) @ dequant(b[e])^T
// (flashinfer.grouped_mm.grouped_mm_bf16, formula, with the operand format of
// flashinfer.gemm.mm_nvfp4_lora).  Same wavefront blocks and K loop as above;
// the tiles are cut per expert from a device-side scan of m_indptr (none
// padded in memory): 256-row tiles, and a 128 x 512 tile for a last piece of
// at most 128 rows, so an expert pads at most 127 rows.
// ---------------------------------------------------------------------------
constexpr int NVG_MAX_EXPERTS = 1024;

template <typename OutT>
struct NvgArgs {
  const uint8_t* a;
  const uint8_t* a_sf;
  const uint8_t* b;
  const uint8_t* b_sf;
  const int32_t* m_indptr;
  const float* alpha;  // [E]
  OutT* out;
  int m_rows, n, k, E;
  uint32_t b_sf_per;  // bytes of one expert's scale buffer
};

__device__ __forceinline__ void nvg_store(uint16_t* p, float v) {
  *p = static_cast<uint16_t>(f32_to_bf16_rne(v));
}
__device__ __forceinline__ void nvg_store(float* p, float v) { *p = v; }
// 4 consecutive outputs, one rounding each: 8 bytes (bf16) or 16 bytes (fp32)
__device__ __forceinline__ void nvg_store4(uint16_t* p, f32x4 v) {
  *reinterpret_cast<u32x2*>(p) = u32x2{f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                                       f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16)};
}
__device__ __forceinline__ void nvg_store4(float* p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}

template <typename OutT>
__global__ __launch_bounds__(NV_NT, 1) void nvfp4_grouped_kernel(NvgArgs<OutT> p) {
  constexpr int FM = 4, FN = 4;                  // 32x32 blocks per wavefront (128 x 128)
  __shared__ int s_full0[NVG_MAX_EXPERTS + 1];  // first 256-row tile of each expert
  __shared__ int s_half0[NVG_MAX_EXPERTS + 1];  // first 128-row tile of each expert
  __shared__ int s_row0[NVG_MAX_EXPERTS + 1];   // clamped first row (s_row0[E]: the end)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = p.E;
  // 128-row tiles (for an expert's last piece of at most 128 rows) span 512
  // columns, so every wavefront keeps its 128 x 128 block; they need n % 512 == 0
  const bool halves = (p.n & 511) == 0;

  // ---- device-side walk of m_indptr (wavefront 0): per expert, the number of
  // 256-row tiles and whether its last piece is a 128-row tile ----
  auto pieces = [&](int len, int& nf, int& nh) {
    const int q = len >> 8, r = len & 255;
    const bool h = halves && r > 0 && r <= 128;
    nf = q + (r > 0 && !h);
    nh = h;
  };
  if (wave == 0) {
    const int per = (E + 63) / 64;
    const int e0 = lane * per;
    int lf = 0, lh = 0;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < E) {
        const int s = min(max(p.m_indptr[e], 0), p.m_rows);
        const int t = min(max(p.m_indptr[e + 1], s), p.m_rows);
        s_row0[e] = s;
        int nf, nh;
        pieces(t - s, nf, nh);
        lf += nf;
        lh += nh;
      }
    }
    int inf = lf, inh = lh;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int vf = __shfl_up(inf, off, 64), vh = __shfl_up(inh, off, 64);
      if (lane >= off) {
        inf += vf;
        inh += vh;
      }
    }
    int rf = inf - lf, rh = inh - lh;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < E) {
        s_full0[e] = rf;
        s_half0[e] = rh;
        const int s = s_row0[e];
        const int t = min(max(p.m_indptr[e + 1], s), p.m_rows);
        int nf, nh;
        pieces(t - s, nf, nh);
        rf += nf;
        rh += nh;
      }
    }
    if (lane == 63) {
      s_full0[E] = inf;
      s_half0[E] = inh;
      s_row0[E] = min(max(p.m_indptr[E], 0), p.m_rows);
    }
  }
  __syncthreads();

  // ---- tile of this workgroup.  The 256-row tiles (256-column panels) come
  // first, then the 128-row ones (512-column panels); each list in grouped
  // order is cut into 8 contiguous runs, one per XCD: an XCD's first run_f
  // workgroups take its run of the first list, the next run_h its run of the
  // second ----
  const int cnt_f = s_full0[E], cnt_h = s_half0[E];
  const int nt_f = p.n / NV_BN, nt_h = p.n / (2 * NV_BN);
  const long total_f = static_cast<long>(cnt_f) * nt_f, total_h = static_cast<long>(cnt_h) * nt_h;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const long run_f = (total_f + 7) / 8, run_h = (total_h + 7) / 8;
  const bool half = slot >= run_f;
  const long L = half ? xcd * run_h + (slot - run_f) : xcd * run_f + slot;
  if (half ? (slot - run_f >= run_h || L >= total_h) : L >= total_f) return;
  const int cnt = half ? cnt_h : cnt_f, nt = half ? nt_h : nt_f;
  const long span = static_cast<long>(NV_GROUP_M) * nt;
  const int grp = static_cast<int>(L / span), first = grp * NV_GROUP_M;
  const int gsize = min(cnt - first, NV_GROUP_M);
  const int in_grp = static_cast<int>(L - grp * span);
  const int mt = first + in_grp % gsize, ni = in_grp / gsize;
  const int* pre = half ? s_half0 : s_full0;
  int lo = 0, hi = E;  // expert of list entry mt: pre[lo] <= mt < pre[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= mt) lo = mid; else hi = mid;
  }
  const int e = __builtin_amdgcn_readfirstlane(lo);
  // a 128-row tile is the expert's last piece, after its 256-row tiles
  const int m0 = __builtin_amdgcn_readfirstlane(
      s_row0[e] + (half ? s_full0[e + 1] - s_full0[e] : mt - s_full0[e]) * NV_BM);
  const int m_end = __builtin_amdgcn_readfirstlane(max(s_row0[e + 1], s_row0[e]));
  // wavefront block: rows m0 + wm*128, columns n0 + wn*128
  const int wm = half ? 0 : wave / NV_WN, wn = half ? wave : wave % NV_WN;
  const int n0 = ni * (half ? 2 * NV_BN : NV_BN);

  // ---- operands: a rows clamped into the expert's rows; b, b_sf of expert e ----
  const int r32 = lane & 31, h = lane >> 5;
  const uint32_t kb = static_cast<uint32_t>(p.k) / 2;
  const int nct = (p.k / 16 + 3) / 4;
  NvOps op;
  op.ra = buf_rsrc(p.a, static_cast<uint32_t>(p.m_rows) * kb);
  op.rb = buf_rsrc(p.b + static_cast<long>(e) * p.n * kb, static_cast<uint32_t>(p.n) * kb);
  op.rsa = buf_rsrc(p.a_sf, static_cast<uint32_t>((p.m_rows + 127) / 128) * nct * 512);
  op.rsb = buf_rsrc(p.b_sf + static_cast<long>(e) * p.b_sf_per, p.b_sf_per);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int row = min(m0 + wm * 128 + i * 32 + r32, m_end - 1);
    op.oa[i] = static_cast<uint32_t>(row) * kb + h * 32;
    op.osa[i] = static_cast<uint32_t>(sf_tile_word(row, h, nct));
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int row = n0 + wn * 128 + j * 32 + r32;
    op.ob[j] = static_cast<uint32_t>(row) * kb + h * 32;
    op.osb[j] = static_cast<uint32_t>(sf_tile_word(row, h, nct));
  }

  f32x16 acc[FM][FN];
  nv_kloop(acc, op, p.k / NV_KC);

  // ---- epilogue: alpha[e] * acc, one rounding; rows past the expert's end dropped ----
  if (m0 + wm * 128 >= m_end) return;
  const float alpha = p.alpha[e];
  // 4 consecutive columns per store where out is aligned for it (n % 256 == 0)
  const bool vec = (reinterpret_cast<uintptr_t>(p.out) & (4 * sizeof(OutT) - 1)) == 0;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int row = m0 + wm * 128 + i * 32 + r32;
    if (row >= m_end) continue;
    OutT* orow = p.out + static_cast<long>(row) * p.n;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = n0 + wn * 128 + j * 32 + 8 * g + 4 * h;
        const f32x4 v = {__fmul_rn(alpha, acc[i][j][4 * g]), __fmul_rn(alpha, acc[i][j][4 * g + 1]),
                         __fmul_rn(alpha, acc[i][j][4 * g + 2]),
                         __fmul_rn(alpha, acc[i][j][4 * g + 3])};
        if (vec) {
          nvg_store4(orow + c0, v);
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) nvg_store(orow + c0 + c, v[c]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fold: b_folded = bf16_rne(fp32(lora_b) * (lora_scale / alpha)), flag
// ---------------------------------------------------------------------------
__global__ void fold_kernel(const uint16_t* __restrict__ lora_b, long count,
                            const float* __restrict__ lora_scale, const float* __restrict__ alpha,
                            uint16_t* __restrict__ b_folded, uint32_t* __restrict__ flags) {
  const float s = lora_scale[0];
  const float ratio = __fdiv_rn(s, alpha[0]);  // IEEE division, round to nearest even
  const long i0 = (static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x) * 8;
  if (i0 == 0) flags[0] = (s == 0.f) ? 1u : 0u;
  if (i0 >= count) return;
  if (i0 + 8 <= count) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(lora_b + i0);
    u32x4 o;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float lo = __fmul_rn(bf16_bits_to_f32(v[c] & 0xffffu), ratio);
      const float hi = __fmul_rn(bf16_bits_to_f32(v[c] >> 16), ratio);
      o[c] = f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
    }
    *reinterpret_cast<u32x4*>(b_folded + i0) = o;
  } else {
    for (long i = i0; i < count; ++i)
      b_folded[i] =
          static_cast<uint16_t>(f32_to_bf16_rne(__fmul_rn(bf16_bits_to_f32(lora_b[i]), ratio)));
  }
}

// ---------------------------------------------------------------------------
// dequant: one thread per 8 codes of one row, with the GEMM's decoder (the
// same scale-word conversion, scale selection and code conversion as the K
// loop)
// ---------------------------------------------------------------------------
__global__ void dequant_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ sf,
                               int rows, int k, uint16_t* __restrict__ out) {
  const long idx = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int words = k / 8;
  if (idx >= static_cast<long>(rows) * words) return;
  const int row = static_cast<int>(idx / words), w = static_cast<int>(idx % words);
  const int col = w / 2;  // 8 elements per word, 16 per scale
  const int n_col_tiles = (k / 16 + 3) / 4;
  const uint32_t sword =
      *reinterpret_cast<const uint32_t*>(sf + sf_tile_word(row, col >> 2, n_col_tiles));
  f16x2 s01, s23;
  ue4m3x4_to_f16(sword, s01, s23);
  const uint32_t cw = *reinterpret_cast<const uint32_t*>(codes + static_cast<long>(row) * (k / 2) + w * 4);
  const u32x4 h = decode8(cw, scale_splat(s01, s23, col & 3));
  u32x4 o;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    o[c] = f16_to_bf16_bits(h[c] & 0xffffu) | (f16_to_bf16_bits(h[c] >> 16) << 16);
  *reinterpret_cast<u32x4*>(out + static_cast<long>(row) * k + w * 8) = o;
}

size_t sf_needed(int64_t rows, int64_t k) {
  return static_cast<size_t>((rows + 127) / 128) * static_cast<size_t>((k / 16 + 3) / 4) * 512;
}

}  // namespace
}  // namespace mi

extern "C" mi_status mi_mm_nvfp4_lora(const uint8_t* a, const uint8_t* b, const uint8_t* a_sf,
                                      size_t a_sf_bytes, const uint8_t* b_sf, size_t b_sf_bytes,
                                      const float* alpha, int64_t m, int64_t n, int64_t k,
                                      const void* d, int64_t rank, const void* lora_b,
                                      const float* lora_scale, const void* b_folded,
                                      const uint32_t* fold_flags, const void* bias, void* out,
                                      void* stream) {
  using namespace mi;
  clear_error();
  MI_REQUIRE(m >= 1, "mm_nvfp4_lora: M >= 1 required (got %lld)", (long long)m);
  MI_REQUIRE(n >= 1, "mm_nvfp4_lora: N >= 1 required (got %lld)", (long long)n);
  MI_REQUIRE(k >= 256 && k % 256 == 0, "mm_nvfp4_lora: K must be a multiple of 256 (got %lld)",
             (long long)k);
  MI_REQUIRE(m < (1LL << 31) && n < (1LL << 31) && k < (1LL << 31) && m * n < (1LL << 40),
             "mm_nvfp4_lora: shape too large");
  MI_REQUIRE(a && b && a_sf && b_sf && alpha && out, "mm_nvfp4_lora: a, b, a_sf, b_sf, alpha and "
             "out must be non-null");
  MI_REQUIRE_SUPPORTED(m * (k / 2) < (1LL << 32) && n * (k / 2) < (1LL << 32) &&
                           sf_needed(m, k) < (1ULL << 32) && sf_needed(n, k) < (1ULL << 32),
                       "mm_nvfp4_lora: each operand's codes and scales must stay below 4 GiB");
  MI_REQUIRE(a_sf_bytes >= sf_needed(m, k),
             "mm_nvfp4_lora: a_sf holds %zu bytes, the 128x4 layout needs %zu", a_sf_bytes,
             sf_needed(m, k));
  MI_REQUIRE(b_sf_bytes >= sf_needed(n, k),
             "mm_nvfp4_lora: b_sf holds %zu bytes, the 128x4 layout needs %zu", b_sf_bytes,
             sf_needed(n, k));
  const bool raw = lora_b != nullptr || lora_scale != nullptr;
  const bool prepared = b_folded != nullptr;
  MI_REQUIRE(!(raw && prepared),
             "mm_nvfp4_lora: pass either the raw adapter (lora_b, lora_scale) or the prepared "
             "adapter, not both");
  int mode = 0;
  if (prepared) {
    MI_REQUIRE(d != nullptr, "mm_nvfp4_lora: the prepared path requires d");
    MI_REQUIRE(fold_flags != nullptr, "mm_nvfp4_lora: the prepared adapter needs its fold flags");
    mode = 2;
  } else if (lora_scale != nullptr) {  // lora_scale NULL disables the adapter
    MI_REQUIRE(d != nullptr && lora_b != nullptr,
               "mm_nvfp4_lora: the raw path needs d and lora_b with lora_scale");
    mode = 1;
  }
  if (mode != 0) {
    MI_REQUIRE(rank >= 8 && rank <= 128 && rank % 8 == 0,
               "mm_nvfp4_lora: LoRA rank must be a multiple of 8 in [8, 128] (got %lld)",
               (long long)rank);
    MI_REQUIRE(aligned16(d) && aligned16(mode == 1 ? lora_b : b_folded),
               "mm_nvfp4_lora: d and lora_b rows must be 16-byte aligned");
  }
  MI_REQUIRE(aligned16(a) && aligned16(b), "mm_nvfp4_lora: a and b must be 16-byte aligned");
  MI_REQUIRE((reinterpret_cast<uintptr_t>(a_sf) & 3) == 0 &&
                 (reinterpret_cast<uintptr_t>(b_sf) & 3) == 0,
             "mm_nvfp4_lora: scale buffers must be 4-byte aligned");

  NvArgs args;
  args.a = a;
  args.b = b;
  args.a_sf = a_sf;
  args.b_sf = b_sf;
  args.alpha = alpha;
  args.d = static_cast<const uint16_t*>(d);
  args.lora_b = static_cast<const uint16_t*>(lora_b);
  args.lora_scale = lora_scale;
  args.b_folded = static_cast<const uint16_t*>(b_folded);
  args.fold_flags = fold_flags;
  args.bias = static_cast<const uint16_t*>(bias);
  args.out = static_cast<uint16_t*>(out);
  args.m = static_cast<int>(m);
  args.n = static_cast<int>(n);
  args.k = static_cast<int>(k);
  args.rank = static_cast<int>(rank);
  args.mode = mode;
  const long tiles = ((m + NV_BM - 1) / NV_BM) * ((n + NV_BN - 1) / NV_BN);
  const long grid = ((tiles + 7) / 8) * 8;
  hipLaunchKernelGGL(nvfp4_lora_kernel, dim3(grid), dim3(NV_NT), 0,
                     static_cast<hipStream_t>(stream), args);
  return launch_status("mm_nvfp4_lora");
}

extern "C" mi_status mi_prepare_lora_fold(const void* lora_b, int64_t n, int64_t rank,
                                          const float* lora_scale, const float* alpha,
                                          void* b_folded, uint32_t* fold_flags, void* stream) {
  using namespace mi;
  clear_error();
  MI_REQUIRE(n >= 1 && rank >= 1, "prepare_lora_fold: N and rank must be >= 1");
  MI_REQUIRE(lora_b && lora_scale && alpha && b_folded && fold_flags,
             "prepare_lora_fold: null pointer argument");
  MI_REQUIRE(lora_b != b_folded, "prepare_lora_fold: b_folded may not alias lora_b");
  MI_REQUIRE(aligned16(lora_b) && aligned16(b_folded),
             "prepare_lora_fold: lora_b and b_folded must be 16-byte aligned");
  const long count = n * rank;
  const long threads = (count + 7) / 8;
  const int block = 256;
  const long grid = (threads + block - 1) / block;
  hipLaunchKernelGGL(fold_kernel, dim3(grid), dim3(block), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(lora_b), count, lora_scale, alpha,
                     static_cast<uint16_t*>(b_folded), fold_flags);
  return launch_status("prepare_lora_fold");
}

extern "C" mi_status mi_nvfp4_dequant_bf16(const uint8_t* codes, const uint8_t* sf,
                                           size_t sf_bytes, int64_t rows, int64_t k, void* out,
                                           void* stream) {
  using namespace mi;
  clear_error();
  MI_REQUIRE(rows >= 1 && rows < (1LL << 31), "nvfp4_dequant: rows must be >= 1");
  MI_REQUIRE(k >= 64 && k % 64 == 0 && k < (1LL << 31), "nvfp4_dequant: K %% 64 == 0 required");
  MI_REQUIRE(codes && sf && out, "nvfp4_dequant: null pointer argument");
  MI_REQUIRE(sf_bytes >= sf_needed(rows, k), "nvfp4_dequant: scale buffer too small");
  MI_REQUIRE(aligned16(out) && (reinterpret_cast<uintptr_t>(codes) & 3) == 0 &&
                 (reinterpret_cast<uintptr_t>(sf) & 3) == 0,
             "nvfp4_dequant: out must be 16-byte aligned, codes and sf 4-byte aligned");
  const long threads = rows * (k / 8);
  const int block = 256;
  hipLaunchKernelGGL(dequant_kernel, dim3((threads + block - 1) / block), dim3(block), 0,
                     static_cast<hipStream_t>(stream), codes, sf, static_cast<int>(rows),
                     static_cast<int>(k), static_cast<uint16_t*>(out));
  return launch_status("nvfp4_dequant");
}

extern "C" mi_status mi_grouped_mm_nvfp4(const uint8_t* a, const uint8_t* a_sf, size_t a_sf_bytes,
                                         int64_t m_rows, int64_t k, const uint8_t* b,
                                         const uint8_t* b_sf, size_t b_sf_bytes, int64_t batch,
                                         int64_t n, const int32_t* m_indptr, const float* alpha,
                                         void* out, mi_dtype out_dtype, void* stream) {
  using namespace mi;
  clear_error();
  MI_REQUIRE(batch >= 1 && batch <= NVG_MAX_EXPERTS,
             "grouped_mm_nvfp4: batch_size must be in [1, %d] (got %lld)", NVG_MAX_EXPERTS,
             (long long)batch);
  MI_REQUIRE(m_rows >= 0 && m_rows < (1LL << 31), "grouped_mm_nvfp4: cum_m out of range");
  MI_REQUIRE(n > 0 && n % 256 == 0 && n < (1LL << 31),
             "grouped_mm_nvfp4: n %% 256 == 0 required (got n=%lld)", (long long)n);
  MI_REQUIRE(k >= 256 && k % 256 == 0 && k < (1LL << 31),
             "grouped_mm_nvfp4: K must be a multiple of 256 (got %lld)", (long long)k);
  MI_REQUIRE(out_dtype == MI_BF16 || out_dtype == MI_F32,
             "grouped_mm_nvfp4: out_dtype must be bf16 or fp32");
  MI_REQUIRE(m_indptr != nullptr && alpha != nullptr && b != nullptr && b_sf != nullptr,
             "grouped_mm_nvfp4: m_indptr, alpha, b and b_sf must be non-null");
  MI_REQUIRE_SUPPORTED(m_rows * (k / 2) < (1LL << 32) && n * (k / 2) < (1LL << 32) &&
                           sf_needed(m_rows, k) < (1ULL << 32),
                       "grouped_mm_nvfp4: a's codes and scales and one expert's codes must stay "
                       "below 4 GiB");
  const size_t per = sf_needed(n, k);
  MI_REQUIRE(b_sf_bytes >= per * static_cast<size_t>(batch),
             "grouped_mm_nvfp4: b_sf holds %zu bytes, %lld experts' 128x4 layouts need %zu",
             b_sf_bytes, (long long)batch, per * static_cast<size_t>(batch));
  if (m_rows == 0) return MI_OK;
  MI_REQUIRE(a != nullptr && a_sf != nullptr && out != nullptr,
             "grouped_mm_nvfp4: a, a_sf and out must be non-null");
  MI_REQUIRE(a_sf_bytes >= sf_needed(m_rows, k),
             "grouped_mm_nvfp4: a_sf holds %zu bytes, the 128x4 layout needs %zu", a_sf_bytes,
             sf_needed(m_rows, k));
  MI_REQUIRE(aligned16(a) && aligned16(b), "grouped_mm_nvfp4: a and b must be 16-byte aligned");
  MI_REQUIRE((reinterpret_cast<uintptr_t>(a_sf) & 3) == 0 &&
                 (reinterpret_cast<uintptr_t>(b_sf) & 3) == 0,
             "grouped_mm_nvfp4: scale buffers must be 4-byte aligned");
  // slots per XCD: both lists' runs (each at most ceil(tiles / 8))
  const long ub = ((m_rows + NV_BM - 1) / NV_BM + batch) * (n / NV_BN);
  const long grid = ((ub + 7) / 8 + 2) * 8;
  MI_REQUIRE(grid < (1L << 31), "grouped_mm_nvfp4: problem too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto fill = [&](auto& args, auto* o) {
    args.a = a;
    args.a_sf = a_sf;
    args.b = b;
    args.b_sf = b_sf;
    args.m_indptr = m_indptr;
    args.alpha = alpha;
    args.out = o;
    args.m_rows = static_cast<int>(m_rows);
    args.n = static_cast<int>(n);
    args.k = static_cast<int>(k);
    args.E = static_cast<int>(batch);
    args.b_sf_per = static_cast<uint32_t>(per);
  };
  if (out_dtype == MI_BF16) {
    NvgArgs<uint16_t> args;
    fill(args, static_cast<uint16_t*>(out));
    hipLaunchKernelGGL(nvfp4_grouped_kernel<uint16_t>, dim3(grid), dim3(NV_NT), 0, s, args);
  } else {
    NvgArgs<float> args;
    fill(args, static_cast<float*>(out));
    hipLaunchKernelGGL(nvfp4_grouped_kernel<float>, dim3(grid), dim3(NV_NT), 0, s, args);
  }
  return launch_status("grouped_mm_nvfp4");
}
