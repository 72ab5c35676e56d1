// Ragged per-expert grouped GEMM on gfx950 bf16 MFMA.
//
// Computes, for every expert e with s = m_indptr[e], t = m_indptr[e+1],
//   out[s:t] = a[s:t] @ b[e]^T
// (flashinfer.grouped_mm.grouped_mm_bf16, formula).  The expert boundaries are
// read on the device only: each workgroup scans m_indptr into LDS, turns it
// into per-expert counts of BM-row tiles, and walks a flat tile index through
// that table -- empty experts own no tile and no row is padded in memory
// (the device-walk backend's behaviour described on the same page).
//
// Three kernels, chosen from host sizes: for groups averaging fewer than 192
// rows grouped_mm_dma64_kernel; for larger ones grouped_mm_dma_kernel when
// n % 512 == 0 and grouped_mm_big_kernel otherwise (each with its own notes
// below).  FC1 takes the same two large-group kernels with the SwiGLU
// activation in their epilogue (gate and up rows paired inside each
// wavefront); it does not use the small-group kernel.
#include "common.hpp"

namespace mi {
namespace {

constexpr int GM_MAX_EXPERTS = 1024;
constexpr int GM_GROUP_M = 8;

// output element types: bf16 bits, fp16, fp32; one rounding to nearest even
struct Bf16Out { uint16_t bits; };
// the MFMA for the input type: bf16 or fp16 operands, fp32 accumulation
template <bool F16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Large groups: 256-column tiles of 256 or 128 rows, four wavefronts of 128
// rows each (one per SIMD), one tile per workgroup.
//
// Tiles.  Every expert's rows are cut into 256-row tiles; a last piece of at
// most 128 rows becomes a 128-row tile instead, which takes about half the
// time (at most 127 padded rows per expert instead of 255).  The 256-row tiles
// come first in the walk and the 128-row ones after; each list, in grouped
// order (GM_GROUP_M m-tiles sweep each n-panel together), is cut into 8
// contiguous runs, one per XCD, so the XCDs get equal work and each keeps its
// a and b panels in its own L2.
//
// K loop.  Per 64-wide K step every wavefront runs 4 sub-steps of
// v_mfma_f32_32x32x16 blocks (4 x FN of them).  The fragments of sub-step s+1
// are read from LDS while the MFMAs of sub-step s run (two fragment register
// sets), so with one wavefront per SIMD the LDS latency stays hidden.  The K
// step's one barrier sits before the last sub-step's MFMAs, and the next
// stage's first fragments are read right after it, under those MFMAs.  Global
// loads run GB_P K steps ahead in registers; the next stage is copied to the
// other LDS buffer during sub-step 1.  LDS rows are padded to 72 elements
// (144 bytes): the 32 rows of a fragment read and the 8 chunks of a row write
// both spread over all banks.
// ---------------------------------------------------------------------------
constexpr int GB_BN = 256, GB_BK = 64;
constexpr int GB_P = 2;   // K steps of global loads in flight, 256-row tiles
constexpr int GB_PH = 2;  // the same for 128-row tiles
constexpr int GB_RS = GB_BK + 8;                 // padded LDS row (16-bit elements)
constexpr int GB_STAGE = (256 + GB_BN) * GB_RS;  // elements per LDS stage (largest tile)

// Device-side walk of m_indptr by wavefront 0: the clamped first row of every
// expert (s_row0[E] = the end of the last one), the first 256-row tile
// (s_full0) and the first 128-row tile (s_half0) of each expert.
__device__ __forceinline__ void gb_walk(const int32_t* __restrict__ m_indptr, int m_rows, int E,
                                        int* s_full0, int* s_half0, int* s_row0) {
  const int lane = threadIdx.x & 63;
  const int per = (E + 63) / 64;
  const int e0 = lane * per;
  int nf = 0, nh = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) {
      const int s = min(max(m_indptr[e], 0), m_rows);
      const int t = min(max(m_indptr[e + 1], s), m_rows);
      s_row0[e] = s;
      const int q = (t - s) >> 8, r = (t - s) & 255;
      nf += q + (r > 128);
      nh += (r > 0 && r <= 128);
    }
  }
  int incl_f = nf, incl_h = nh;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int vf = __shfl_up(incl_f, off, 64), vh = __shfl_up(incl_h, off, 64);
    if (lane >= off) {
      incl_f += vf;
      incl_h += vh;
    }
  }
  int run_f = incl_f - nf, run_h = incl_h - nh;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) {
      s_full0[e] = run_f;
      s_half0[e] = run_h;
      const int s = s_row0[e];
      const int t = min(max(m_indptr[e + 1], s), m_rows);
      const int q = (t - s) >> 8, r = (t - s) & 255;
      run_f += q + (r > 128);
      run_h += (r > 0 && r <= 128);
    }
  }
  if (lane == 63) {
    s_full0[E] = incl_f;
    s_half0[E] = incl_h;
    s_row0[E] = min(max(m_indptr[E], 0), m_rows);
  }
}

// m-tile and n-panel of linear index L in the grouped order of a list of
// `count` m-tiles
__device__ __forceinline__ void gb_order(long L, int count, int nt, int& mt, int& ni) {
  const long span = static_cast<long>(GM_GROUP_M) * nt;
  const int grp = static_cast<int>(L / span);
  const int first = grp * GM_GROUP_M;
  const int gsize = min(count - first, GM_GROUP_M);
  const int in_grp = static_cast<int>(L - static_cast<long>(grp) * span);
  mt = first + in_grp % gsize;
  ni = in_grp / gsize;
}

// expert owning list entry mt: last e with pre[e] <= mt (pre non-decreasing,
// pre[0] = 0 <= mt < pre[E])
__device__ __forceinline__ int gb_owner(const int* pre, int E, int mt) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= mt) lo = mid; else hi = mid;
  }
  return lo;
}

// four consecutive output columns of one row: one buffer store at byte offset
// `off`; a store past the descriptor's range is dropped
template <typename OutT>
__device__ __forceinline__ void bstore_out4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v);
template <>
__device__ __forceinline__ void bstore_out4<Bf16Out>(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                     f32x4 v) {
  typedef __bf16 b4 __attribute__((ext_vector_type(4)));
  // hardware conversion: round to nearest even
  const b4 h = __builtin_convertvector(v, b4);
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h), r, off, 0, 0);
}
template <>
__device__ __forceinline__ void bstore_out4<_Float16>(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                      f32x4 v) {
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  const h4 h = __builtin_convertvector(v, h4);
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h), r, off, 0, 0);
}
template <>
__device__ __forceinline__ void bstore_out4<float>(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                   f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
}

// 4 outputs converted to OutT and packed (the conversions of bstore_out4)
template <typename OutT>
struct Packed4;
template <>
struct Packed4<Bf16Out> {
  typedef u32x2 T;
  __device__ static T pack(f32x4 v) {
    typedef __bf16 b4 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(u32x2, __builtin_convertvector(v, b4));
  }
};
template <>
struct Packed4<_Float16> {
  typedef u32x2 T;
  __device__ static T pack(f32x4 v) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(u32x2, __builtin_convertvector(v, h4));
  }
};
template <>
struct Packed4<float> {
  typedef u32x4 T;
  __device__ static T pack(f32x4 v) { return __builtin_bit_cast(u32x4, v); }
};

// Instruction interleave of a sub-step: the NR LDS reads of the next
// fragments go out between the first NR of its NM MFMAs, so they complete
// under this sub-step.
template <int NR, int NM>
__device__ __forceinline__ void gb_interleave_reads() {
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
}
// sub-step 1 also copies the next stage to LDS (NC writes) and refills its
// register slot (NC global loads), spread over the remaining MFMAs
template <int NR, int NM, int NC>
__device__ __forceinline__ void gb_interleave_copy() {
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
  }
  constexpr int REST = NM - NR, PER = (NC + REST - 1) / REST;
#pragma unroll
  for (int i = 0; i < REST; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x200, PER, 0);  // LDS write
    __builtin_amdgcn_sched_group_barrier(0x020, PER, 0);  // global load
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
  }
}

// FC1 epilogue parameters: the gate/up halves of b and the SwiGLU activation
struct GbGlu {
  const uint16_t* delta;  // bf16 [m_rows, 2I] added before the activation, or null
  const float* alpha;     // [E] or null (1)
  const float* beta;      // [E] or null (0)
  const float* limit;     // [E] or null (no clamp)
};

// One output tile: 256 rows (FN = 4: waves 2 x 2, 128 x 128 each) or 128 rows
// (FN = 2: waves 1 x 4, 128 x 64 each), 256 columns.  `rows` (1..BM) of the
// tile belong to the expert; the a descriptor covers only those, so rows past
// them read as zero and their stores are dropped.
//
// GLU (FC1): b[e] is [n = 2I, k], gate rows 0..I-1 and up rows I..2I-1.  A
// tile then covers 128 output columns c0 = n0/2 ..: each wavefront's b
// fragments j < FN/2 are gate rows and j >= FN/2 the matching up rows, so one
// lane holds both operands of every output it writes; out is [m_rows, I].
template <int FN, int P, bool F16, bool GLU, typename OutT>
__device__ __forceinline__ void gb_tile(const uint16_t* __restrict__ a,
                                        const uint16_t* __restrict__ b, OutT* __restrict__ out,
                                        uint16_t* smem, int e, int m0, int rows, int n0, int k,
                                        int n, const GbGlu& gl) {
  constexpr int WN = FN == 4 ? 2 : 4;        // wavefronts along n
  constexpr int BM = 128 * (4 / WN);         // tile rows
  constexpr int CPT_A = BM / 32, CPT_B = 8;  // 16-byte chunks per thread per stage
  constexpr int NR = 4 + FN, NM = 4 * FN;    // fragment reads and MFMAs per sub-step
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int r = lane & 31, h = lane >> 5;
  const int KT = k / GB_BK;
  const uint32_t kbytes = static_cast<uint32_t>(k) * 2;

  const __amdgpu_buffer_rsrc_t ar = buf_rsrc(a + static_cast<long>(m0) * k, rows * kbytes);
  const int inter = n / 2, c0 = n0 / 2;  // GLU: output width and first output column
  const long b_row0 = static_cast<long>(e) * n + (GLU ? c0 : n0);
  const __amdgpu_buffer_rsrc_t br = buf_rsrc(
      b + b_row0 * k, static_cast<uint32_t>(GLU ? inter + 128 : GB_BN) * kbytes);
  // b row (relative to b_row0) of staging block i (LDS rows 32i .. 32i+31)
  uint32_t b_so[CPT_B];
#pragma unroll
  for (int i = 0; i < CPT_B; ++i) {
    int row = 32 * i;
    if constexpr (GLU) {
      const int jj = i % FN;  // fragment of wavefront i / FN
      row = (jj < FN / 2 ? 0 : inter) + (i / FN) * 16 * FN + (jj % (FN / 2)) * 32;
    }
    b_so[i] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(row) * kbytes);
  }

  // staging: chunk c = tid + 256 i is row c/8 = tid/8 + 32 i, 16-byte chunk
  // tid%8 of the stage
  const uint32_t g_off = static_cast<uint32_t>(tid >> 3) * kbytes + (tid & 7) * 16;
  const uint32_t g_step = 32 * kbytes;  // 32 rows
  const int st_lds = (tid >> 3) * GB_RS + (tid & 7) * 8;
  // fragments: lane (r, h) reads row r of each 32-row block, 16-byte chunk 2s+h
  const int fa_base = (wm * 128 + r) * GB_RS + 8 * h;
  const int fb_base = 256 * GB_RS + (wn * 32 * FN + r) * GB_RS + 8 * h;

  f32x16 acc[4][FN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  struct Frag {
    u32x4 a[4], b[FN];
  };
  u32x4 ra[P][CPT_A], rb[P][CPT_B];
  auto gload = [&](int p, int kt) {
    // stages past the end reload the last one: every step issues the same loads
    const uint32_t so = static_cast<uint32_t>(min(kt, KT - 1)) * (GB_BK * 2);
#pragma unroll
    for (int i = 0; i < CPT_A; ++i) ra[p][i] = buf_ld128(ar, g_off + i * g_step, so);
#pragma unroll
    for (int i = 0; i < CPT_B; ++i) rb[p][i] = buf_ld128(br, g_off, so + b_so[i]);
  };
  auto lstore = [&](int p, uint16_t* st) {
#pragma unroll
    for (int i = 0; i < CPT_A; ++i)
      *reinterpret_cast<u32x4*>(st + st_lds + i * 32 * GB_RS) = ra[p][i];
#pragma unroll
    for (int i = 0; i < CPT_B; ++i)
      *reinterpret_cast<u32x4*>(st + 256 * GB_RS + st_lds + i * 32 * GB_RS) = rb[p][i];
  };
  auto fload = [&](Frag& f, const uint16_t* st, int s) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f.a[i] = *reinterpret_cast<const u32x4*>(st + fa_base + i * 32 * GB_RS + 16 * s);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      f.b[j] = *reinterpret_cast<const u32x4*>(st + fb_base + j * 32 * GB_RS + 16 * s);
  };
  // C[m][n] with m = output column (b row), n = output row (a row)
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<F16>(f.b[j], f.a[i], acc[i][j]);
  };

  Frag f0, f1;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    gload(p, p);
    __builtin_amdgcn_sched_barrier(0);  // slots in order: the loop's waits stay exact
  }
  lstore(0, smem);
  gload(0, P);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  fload(f0, smem, 0);

  // one K step; `q` = register slot holding stage kt+1
  auto kstep = [&](int kt, int q) {
    uint16_t* st = smem + (kt & 1) * GB_STAGE;
    uint16_t* nx = smem + ((kt & 1) ^ 1) * GB_STAGE;
    fload(f1, st, 1);
    mma(f0);
    gb_interleave_reads<NR, NM>();
    __builtin_amdgcn_sched_barrier(0);
    fload(f0, st, 2);
    lstore(q, nx);
    gload(q, kt + 1 + P);
    mma(f1);
    gb_interleave_copy<NR, NM, CPT_A + CPT_B>();
    __builtin_amdgcn_sched_barrier(0);
    fload(f1, st, 3);
    mma(f0);
    gb_interleave_reads<NR, NM>();
    __builtin_amdgcn_sched_barrier(0);
    // every wavefront's LDS work of this step is done: the next stage is
    // complete and this one may be overwritten one step later
    __syncthreads();
    fload(f0, nx, 0);
    mma(f1);
    gb_interleave_reads<NR, NM>();
    __builtin_amdgcn_sched_barrier(0);
  };
  // The loop body is straight-line code (all MFMAs unconditional: rows past
  // the group's end are zeros), so the compiler's wait counts stay exact.
  // register slot (kt + 1) % P holds stage kt + 1
  int kt = 0;
  for (; kt + P <= KT; kt += P) {
#pragma unroll
    for (int q = 0; q < P; ++q) kstep(kt + q, (q + 1) % P);
  }
#pragma unroll
  for (int q = 0; q < P - 1; ++q)
    if (kt + q < KT) kstep(kt + q, (q + 1) % P);

  if (wm * 128 >= rows) return;  // all of this wavefront's rows lie past the group's end
  if constexpr (!GLU) {
    // acc[i][j][q]: tile row wm*128 + i*32 + r, column wn*32*FN + j*32 + 8*(q/4) + 4h + q%4.
    const __amdgpu_buffer_rsrc_t orsrc = buf_rsrc(out + static_cast<long>(m0) * n,
                                                  static_cast<uint32_t>(rows) * n * sizeof(OutT));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t orow =
          (static_cast<uint32_t>(wm * 128 + i * 32 + r) * n + n0 + wn * 32 * FN + 4 * h) *
          sizeof(OutT);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                           acc[i][j][4 * g + 3]};
          bstore_out4<OutT>(orsrc, orow + (j * 32 + 8 * g) * sizeof(OutT), v);
        }
      }
    }
  } else {
    // gate acc[i][j], up acc[i][j + FN/2] (j < FN/2): tile row wm*128 + i*32 + r,
    // output column c0 + wn*16*FN + j*32 + 8*(q/4) + 4h + q%4
    const float alpha = gl.alpha ? gl.alpha[e] : 1.f;
    const float beta = gl.beta ? gl.beta[e] : 0.f;
    const float limit = gl.limit ? gl.limit[e] : __builtin_inff();
    const __amdgpu_buffer_rsrc_t orsrc = buf_rsrc(
        out + static_cast<long>(m0) * inter, static_cast<uint32_t>(rows) * inter * sizeof(OutT));
    const bool has_delta = gl.delta != nullptr;
    const __amdgpu_buffer_rsrc_t drsrc =
        buf_rsrc(has_delta ? gl.delta + static_cast<long>(m0) * n : gl.delta,
                 has_delta ? static_cast<uint32_t>(rows) * n * 2 : 0u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t trow = wm * 128 + i * 32 + r;
#pragma unroll
      for (int j = 0; j < FN / 2; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t col = c0 + wn * 16 * FN + j * 32 + 8 * g + 4 * h;
          float hg[4], hu[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            hg[q] = acc[i][j][4 * g + q];
            hu[q] = acc[i][j + FN / 2][4 * g + q];
          }
          if (has_delta) {
            const u32x2 dg = buf_ld64(drsrc, (trow * n + col) * 2, 0);
            const u32x2 du = buf_ld64(drsrc, (trow * n + inter + col) * 2, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t wg = dg[q >> 1], wu = du[q >> 1];
              hg[q] += __uint_as_float((q & 1) ? (wg & 0xffff0000u) : (wg << 16));
              hu[q] += __uint_as_float((q & 1) ? (wu & 0xffff0000u) : (wu << 16));
            }
          }
          f32x4 v;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float gg = fminf(hg[q], limit);
            const float uu = fminf(fmaxf(hu[q], -limit), limit);
            // logistic function from the hardware exp2 and reciprocal (a few ulp)
            const float sig = __builtin_amdgcn_rcpf(1.f + __expf(-alpha * gg));
            v[q] = gg * sig * (uu + beta);
          }
          bstore_out4<OutT>(orsrc, (trow * inter + col) * sizeof(OutT), v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// grouped_mm_dma_kernel: large groups, n % 512 == 0
//
// What bounds the big tiles is the CU's vector-memory path: every operand
// byte of a tile is a request from the CU's L1 to L2, and the CU sustains
// about 14 bytes of them per clock (the same rate that caps a plain streaming
// read).  Per 64-wide K step a 256 x 256 tile loads 64 KB for 256 MFMAs
// (32x32x16), a 384 x 256 tile 80 KB for 384.  This kernel therefore cuts
// each expert's rows into 384-row tiles, a last piece of 129..256 rows into a
// 256-row tile and of at most 128 rows into a 128-row tile that is 512
// columns wide (128 x 512 loads 80 KB per step for the work of 128 x 256 at
// 48 KB, twice); all three load fewer bytes per MFMA than the 256 x 256 and
// 128 x 256 tiles.
//
// Staging: the tile's a and b rows go straight from memory into LDS
// (buffer_load ... lds: each instruction writes 1 KB, 8 rows of 128 bytes),
// so no registers hold staged data -- the 384-row tile needs them for its
// accumulators.  16-byte chunk c of LDS row R holds the row's chunk
// c ^ gd_swz(R).  Two LDS stages of 80 KB: the loads of step kt+1 are issued
// at the start of step kt and complete by its barrier (one step ahead is as
// fast as two for these tiles).  Eight wavefronts, two per SIMD: 4 x 2 of
// 96 x 128 (384 x 256; four wavefronts of 192 x 128 would need 384
// accumulator registers a lane, which the compiler spills), 2 x 4 of
// 128 x 64 (256 x 256), 1 x 8 of 128 x 64 (128 x 512).  Fragments are
// single-buffered; the SIMD's second wavefront covers the LDS latency.
// ---------------------------------------------------------------------------
constexpr int GD_STAGE = 640 * 64;  // elements per LDS stage: 640 rows of 128 bytes
constexpr int GD_WAVES = 8;         // two wavefronts per SIMD

// Chunk swizzle of LDS row R: any 8 consecutive rows, and the even and the
// odd rows of any 16, take 8 different values (a fragment read of 32 rows
// spreads over all banks whether the LDS serves 8 or 16 lanes a cycle), and it
// depends only on R % 32.
__device__ __forceinline__ int gd_swz(int row) { return (row & 7) ^ ((row >> 3) & 3); }

// an LDS address as the LDS-DMA builtin takes it
typedef __attribute__((address_space(3))) void* lds_void_ptr;
__device__ __forceinline__ lds_void_ptr lds_ptr(uint16_t* p) { return (lds_void_ptr)(p); }

// GLU (FC1): b[e] is [n = 2I, k], gate rows 0..I-1 and up rows I..2I-1, and
// the tile covers BN/2 output columns c0 = n0/2 ..: LDS b block (wn FN + j)
// holds gate rows c0 + wn 16 FN + 32 j .. for j < FN/2 and the matching up rows
// for j >= FN/2, so one lane holds both operands of every output it writes
// (the mapping of grouped_mm_big_kernel); out is [m_rows, I].
// BAUX: cache policy of the b loads (2: non-temporal, streaming).
template <int WM, int WN, int FM, int FN, bool F16, bool GLU, typename OutT, int BAUX = 0>
__device__ __forceinline__ void gd_tile(const uint16_t* __restrict__ a,
                                        const uint16_t* __restrict__ b, OutT* __restrict__ out,
                                        uint16_t* smem, int e, int m0, int rows, int n0, int k,
                                        int n, const GbGlu& gl) {
  constexpr int BM = 32 * FM * WM, BN = 32 * FN * WN;
  constexpr int R = BM + BN;                 // LDS rows per stage
  constexpr int NI = R / 64;                 // DMA instructions per wavefront per stage
  constexpr int NIA = BM / 64;               // of which a rows
  static_assert(WM * WN == GD_WAVES && R <= 640 && BM % 64 == 0, "tile");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int r = lane & 31, h = lane >> 5;
  const int KT = k / GB_BK;
  const uint32_t kbytes = static_cast<uint32_t>(k) * 2;

  const int inter = n / 2, c0 = n0 / 2;  // GLU: output width and first output column
  const __amdgpu_buffer_rsrc_t br =
      buf_rsrc(b + (static_cast<long>(e) * n + (GLU ? c0 : n0)) * k,
               static_cast<uint32_t>(GLU ? inter + BN / 2 : BN) * kbytes);
  static_assert(!GLU || FN % 2 == 0, "GLU pairs gate and up fragments");
  // b row (relative to the descriptor) of the first LDS row of b instruction
  // i >= NIA: LDS b row R = 8 (8i + wave) - BM, block R/32 = wn FN + j
  uint32_t bso[NI - NIA];
#pragma unroll
  for (int i = NIA; i < NI; ++i) {
    const int R = 8 * (8 * i + wave) - BM;
    int row = R;
    if constexpr (GLU) {
      const int blk = R >> 5, jj = blk % FN, wb = blk / FN;
      row = (jj < FN / 2 ? 0 : inter) + wb * 16 * FN + (jj % (FN / 2)) * 32 + (R & 31);
    }
    bso[i - NIA] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(row) * kbytes);
  }

  // DMA instruction i of this wavefront fills LDS rows 8g .. 8g+7 with
  // g = 8i + wave (i < NIA: a rows, else b rows 8g - BM ..).  Lane l takes row
  // 8g + l/8 and its chunk (l%8) ^ gd_swz(8g + l/8) = (l%8) ^ (l/8) ^ (wave%4).
  // Each a instruction has its own descriptor starting at its first row, whose
  // range ends at the group's last row, so rows past the end read as zero (the
  // range check covers the lane offset, which holds the row within the 8).
  const int lr = lane >> 3, lc = lane & 7;
  const uint32_t dvo = static_cast<uint32_t>(lr) * kbytes + ((lc ^ lr ^ (wave & 3)) << 4);
  __amdgpu_buffer_rsrc_t ari[NIA];
#pragma unroll
  for (int i = 0; i < NIA; ++i) {
    const int r0 = 8 * (8 * i + wave);
    ari[i] = buf_rsrc(a + static_cast<long>(m0 + r0) * k,
                      static_cast<uint32_t>(max(rows - r0, 0)) * kbytes);
  }
  auto dma = [&](uint16_t* st, int kt) {
    const uint32_t so = static_cast<uint32_t>(min(kt, KT - 1)) * (GB_BK * 2);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int g = 8 * i + wave;
      uint16_t* dst = st + g * 512;  // 8 rows of 64 elements
      if (i < NIA)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ari[i], lds_ptr(dst), 16, dvo, so, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(br, lds_ptr(dst), 16, dvo, so + bso[i - NIA], 0,
                                                 BAUX);
    }
  };

  // fragments: lane (r, h) reads 16-byte chunk 2s+h of row 32 B + r of each
  // 32-row block B, at slot (2s+h) ^ gd_swz(r)
  int fo[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) fo[s] = r * 64 + (((2 * s + h) ^ gd_swz(r)) << 3);
  struct Frag {
    u32x4 a[FM], b[FN];
  };
  auto fload = [&](Frag& f, const uint16_t* st, int s) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int blk = wm * FM + i;
      f.a[i] = *reinterpret_cast<const u32x4*>(st + blk * 32 * 64 + fo[s]);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int blk = BM / 32 + wn * FN + j;
      f.b[j] = *reinterpret_cast<const u32x4*>(st + blk * 32 * 64 + fo[s]);
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  // C[m][n] with m = output column (b row), n = output row (a row)
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<F16>(f.b[j], f.a[i], acc[i][j]);
  };

  uint16_t* const st0 = smem;
  uint16_t* const st1 = smem + GD_STAGE;
  dma(st0, 0);
  __syncthreads();  // stage 0 in LDS; every wavefront is past the tile walk
  auto kstep = [&](int kt, uint16_t* st, uint16_t* nx) {
    dma(nx, kt + 1);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      Frag f;
      fload(f, st, s);
      mma(f);
    }
    // stage kt+1 has landed (each wavefront waits for its own loads) and every
    // wavefront's reads of stage kt are done
    __syncthreads();
  };
  int kt = 0;
  for (; kt + 2 <= KT; kt += 2) {
    kstep(kt, st0, st1);
    kstep(kt + 1, st1, st0);
  }
  if (kt < KT) kstep(kt, st0, st1);

  // acc[i][j][q]: tile row (wm FM + i) 32 + r, column (wn FN + j) 32 + 8 (q/4) + 4h + q%4
  if (wm * 32 * FM >= rows) return;
  if constexpr (!GLU) {
    const __amdgpu_buffer_rsrc_t orsrc = buf_rsrc(out + static_cast<long>(m0) * n,
                                                  static_cast<uint32_t>(rows) * n * sizeof(OutT));
    // The outputs go through this wavefront's own share of the LDS stages
    // (free after the K loop's last barrier): each lane writes its values in
    // place (one tile row, 4 runs of 4 columns per 32 x 32 block), then reads
    // back 16-byte pieces of whole rows, so each store instruction writes rows
    // of contiguous 16-byte pieces instead of 32 rows of 16 bytes.  Rows past
    // the group's end fall outside the buffer range and are dropped.  The
    // stores are streaming (non-temporal): they now cover whole lines, and the
    // output then does not displace operands from L2 (skewed MoE FC2 1.2-2.4%
    // faster in two interleaved rounds; with 8-byte pieces the same policy was
    // 1.5x slower, since partial lines reached memory uncombined).
    constexpr int ES = sizeof(OutT);
    constexpr int WC = 32 * FN;                         // columns of the wavefront
    constexpr int RB = WC * ES + 16;                    // padded LDS row, bytes
    constexpr int REG = 2 * GD_STAGE * 2 / GD_WAVES;    // LDS bytes per wavefront
    constexpr int PB = REG / (32 * RB) < FM ? REG / (32 * RB) : FM;  // 32-row blocks per pass
    static_assert(PB >= 1, "epilogue stage");
    constexpr int CPR = WC * ES / 16;                   // 16-byte pieces per row
    static_assert(CPR <= 64 && 64 % CPR == 0, "pieces per row");
    constexpr int RPI = 64 / CPR;                       // rows per read instruction
    char* const reg = reinterpret_cast<char*>(smem) + wave * REG;
    const uint32_t col0 = static_cast<uint32_t>(n0 + wn * FN * 32) * ES;
    const int pr = lane / CPR, pc = lane % CPR;
#pragma unroll
    for (int i0 = 0; i0 < FM; i0 += PB) {
#pragma unroll
      for (int ii = 0; ii < PB; ++ii) {
        if (i0 + ii < FM) {
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 v = {acc[i0 + ii][j][4 * g], acc[i0 + ii][j][4 * g + 1],
                               acc[i0 + ii][j][4 * g + 2], acc[i0 + ii][j][4 * g + 3]};
              *reinterpret_cast<typename Packed4<OutT>::T*>(
                  reg + (ii * 32 + r) * RB + (j * 32 + 8 * g + 4 * h) * ES) =
                  Packed4<OutT>::pack(v);
            }
        }
      }
      const int nr = (FM - i0 < PB ? FM - i0 : PB) * 32;  // rows of this pass
#pragma unroll
      for (int rr0 = 0; rr0 < PB * 32; rr0 += RPI) {
        const int rr = rr0 + pr;
        if (rr0 < nr) {
          const u32x4 d = *reinterpret_cast<const u32x4*>(reg + rr * RB + pc * 16);
          const uint32_t trow = static_cast<uint32_t>((wm * FM + i0) * 32 + rr);
          __builtin_amdgcn_raw_buffer_store_b128(d, orsrc, trow * n * ES + col0 + pc * 16, 0, 2);
        }
      }
    }
  } else {
    // gate acc[i][j], up acc[i][j + FN/2] (j < FN/2): tile row (wm FM + i) 32 + r,
    // output column c0 + wn 16 FN + 32 j + 8 (q/4) + 4h + q%4; the SwiGLU of
    // grouped_mm_big_kernel
    const float alpha = gl.alpha ? gl.alpha[e] : 1.f;
    const float beta = gl.beta ? gl.beta[e] : 0.f;
    const float limit = gl.limit ? gl.limit[e] : __builtin_inff();
    const __amdgpu_buffer_rsrc_t orsrc = buf_rsrc(
        out + static_cast<long>(m0) * inter, static_cast<uint32_t>(rows) * inter * sizeof(OutT));
    const bool has_delta = gl.delta != nullptr;
    const __amdgpu_buffer_rsrc_t drsrc =
        buf_rsrc(has_delta ? gl.delta + static_cast<long>(m0) * n : gl.delta,
                 has_delta ? static_cast<uint32_t>(rows) * n * 2 : 0u);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const uint32_t trow = (wm * FM + i) * 32 + r;
#pragma unroll
      for (int j = 0; j < FN / 2; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t col = c0 + wn * 16 * FN + j * 32 + 8 * g + 4 * h;
          float hg[4], hu[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            hg[q] = acc[i][j][4 * g + q];
            hu[q] = acc[i][j + FN / 2][4 * g + q];
          }
          if (has_delta) {
            const u32x2 dg = buf_ld64(drsrc, (trow * n + col) * 2, 0);
            const u32x2 du = buf_ld64(drsrc, (trow * n + inter + col) * 2, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t wg = dg[q >> 1], wu = du[q >> 1];
              hg[q] += __uint_as_float((q & 1) ? (wg & 0xffff0000u) : (wg << 16));
              hu[q] += __uint_as_float((q & 1) ? (wu & 0xffff0000u) : (wu << 16));
            }
          }
          f32x4 v;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float gg = fminf(hg[q], limit);
            const float uu = fminf(fmaxf(hu[q], -limit), limit);
            // logistic function from the hardware exp2 and reciprocal (a few ulp)
            const float sig = __builtin_amdgcn_rcpf(1.f + __expf(-alpha * gg));
            v[q] = gg * sig * (uu + beta);
          }
          bstore_out4<OutT>(orsrc, (trow * inter + col) * sizeof(OutT), v);
        }
      }
    }
  }
}

// Device-side walk of m_indptr by wavefront 0 for the three tile kinds: per
// expert the clamped first row (s_row0[E] = end of the last expert), the
// first 384-row tile (s_t3), 256-row tile (s_t2) and 128-row tile (s_t1).
// An expert of m rows has q = m / 384 full tiles and r = m % 384 rows left:
// r > 256 -> one more 384-row tile, 128 < r <= 256 -> a 256-row tile,
// 0 < r <= 128 -> a 128-row tile.
__device__ __forceinline__ void gd_counts(int m, int& c3, int& c2, int& c1) {
  const int q = m / 384, r = m - 384 * q;
  c3 = q + (r > 256);
  c2 = (r > 128 && r <= 256);
  c1 = (r > 0 && r <= 128);
}
__device__ __forceinline__ void gd_walk(const int32_t* __restrict__ m_indptr, int m_rows, int E,
                                        int* s_t3, int* s_t2, int* s_t1, int* s_row0) {
  const int lane = threadIdx.x & 63;
  const int per = (E + 63) / 64;
  const int e0 = lane * per;
  int n3 = 0, n2 = 0, n1 = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) {
      const int s = min(max(m_indptr[e], 0), m_rows);
      const int t = min(max(m_indptr[e + 1], s), m_rows);
      s_row0[e] = s;
      int c3, c2, c1;
      gd_counts(t - s, c3, c2, c1);
      n3 += c3;
      n2 += c2;
      n1 += c1;
    }
  }
  int i3 = n3, i2 = n2, i1 = n1;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v3 = __shfl_up(i3, off, 64), v2 = __shfl_up(i2, off, 64),
              v1 = __shfl_up(i1, off, 64);
    if (lane >= off) {
      i3 += v3;
      i2 += v2;
      i1 += v1;
    }
  }
  int r3 = i3 - n3, r2 = i2 - n2, r1 = i1 - n1;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) {
      s_t3[e] = r3;
      s_t2[e] = r2;
      s_t1[e] = r1;
      const int s = s_row0[e];
      const int t = min(max(m_indptr[e + 1], s), m_rows);
      int c3, c2, c1;
      gd_counts(t - s, c3, c2, c1);
      r3 += c3;
      r2 += c2;
      r1 += c1;
    }
  }
  if (lane == 63) {
    s_t3[E] = i3;
    s_t2[E] = i2;
    s_t1[E] = i1;
    s_row0[E] = min(max(m_indptr[E], 0), m_rows);
  }
}

template <bool F16, bool GLU, typename OutT>
__global__ __launch_bounds__(64 * GD_WAVES, 1) void grouped_mm_dma_kernel(
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
    const int32_t* __restrict__ m_indptr, OutT* __restrict__ out, int m_rows, int k, int n,
    int E, GbGlu gl) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * GD_STAGE];
  // the walk's tables live in stage 1, which the first K step overwrites only
  // after the barrier that follows stage 0's loads
  int* const s_t3 = reinterpret_cast<int*>(smem + GD_STAGE);
  int* const s_t2 = s_t3 + (GM_MAX_EXPERTS + 1);
  int* const s_t1 = s_t2 + (GM_MAX_EXPERTS + 1);
  int* const s_row0 = s_t1 + (GM_MAX_EXPERTS + 1);

  if ((threadIdx.x >> 6) == 0) gd_walk(m_indptr, m_rows, E, s_t3, s_t2, s_t1, s_row0);
  __syncthreads();

  const int nt = n / 256, nt1 = n / 512;
  const int c3 = s_t3[E], c2 = s_t2[E], c1 = s_t1[E];
  const long tot3 = static_cast<long>(c3) * nt, tot2 = static_cast<long>(c2) * nt,
             tot1 = static_cast<long>(c1) * nt1;
  // The grid is an upper bound on the tiles; the dispatcher deals workgroup
  // ids to the 8 XCDs in turn.  An XCD's first run3 workgroups take its run
  // of the 384-row tiles, the next run2 its 256-row tiles, then run1 its
  // 128-row tiles.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const long run3 = (tot3 + 7) / 8, run2 = (tot2 + 7) / 8, run1 = (tot1 + 7) / 8;
  int kind, e, m0, rows, n0;
  {
    int mt, ni;
    long L;
    if (slot < run3) {
      L = xcd * run3 + slot;
      if (L >= tot3) return;
      gb_order(L, c3, nt, mt, ni);
      e = gb_owner(s_t3, E, mt);
      m0 = s_row0[e] + (mt - s_t3[e]) * 384;
      kind = 3;
      n0 = ni * 256;
    } else if (slot < run3 + run2) {
      L = xcd * run2 + (slot - run3);
      if (L >= tot2) return;
      gb_order(L, c2, nt, mt, ni);
      e = gb_owner(s_t2, E, mt);
      m0 = s_row0[e] + (s_t3[e + 1] - s_t3[e]) * 384;
      kind = 2;
      n0 = ni * 256;
    } else {
      L = xcd * run1 + (slot - run3 - run2);
      if (slot - run3 - run2 >= run1 || L >= tot1) return;
      gb_order(L, c1, nt1, mt, ni);
      e = gb_owner(s_t1, E, mt);
      m0 = s_row0[e] + (s_t3[e + 1] - s_t3[e]) * 384;
      kind = 1;
      n0 = ni * 512;
    }
    const int end = max(s_row0[e + 1], s_row0[e]);
    rows = min(end - m0, kind == 3 ? 384 : kind == 2 ? 256 : 128);
  }
  kind = __builtin_amdgcn_readfirstlane(kind);
  e = __builtin_amdgcn_readfirstlane(e);
  m0 = __builtin_amdgcn_readfirstlane(m0);
  rows = __builtin_amdgcn_readfirstlane(rows);
  n0 = __builtin_amdgcn_readfirstlane(n0);
  if (kind == 3)
    gd_tile<4, 2, 3, 4, F16, GLU, OutT>(a, b, out, smem, e, m0, rows, n0, k, n, gl);
  else if (kind == 2)
    gd_tile<2, 4, 4, 2, F16, GLU, OutT>(a, b, out, smem, e, m0, rows, n0, k, n, gl);
  else
    // an expert's last <= 128 rows: its b panels stream from memory for this
    // one tile, with streaming (non-temporal) loads -- measured on the skewed
    // MoE FC2: the experts under 128 rows alone 567 -> 512 us, the whole call
    // 1443-1450 -> 1414-1415 us, the same output
    gd_tile<1, 8, 4, 2, F16, GLU, OutT, 2>(a, b, out, smem, e, m0, rows, n0, k, n, gl);
}

// ---------------------------------------------------------------------------
// grouped_mm_dma64_kernel: small groups (average < 192 rows): 64 x 128 tiles,
// one per workgroup.  These tiles stream b from memory and are bound by the
// same per-CU L1 -> L2 request rate as the large ones: against 64 x 64 tiles
// they request a quarter fewer operand bytes (a is read once per 128-wide
// n-panel instead of per 64-wide one), with as many tiles as there are CUs on
// the uniform E = 8 x 128-row workload.  a and b rows go straight into LDS
// (the staging of the large-group kernel); four LDS stages of 24 KB, each its
// own array, keep three K steps of loads in flight, which cold data from
// memory needs (one step ahead was measured slower).  8 wavefronts of 32 x 32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void gd64_walk(const int32_t* __restrict__ m_indptr, int m_rows, int E,
                                          int* s_t0, int* s_row0) {
  const int lane = threadIdx.x & 63;
  const int per = (E + 63) / 64;
  const int e0 = lane * per;
  int c = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) {
      const int s = min(max(m_indptr[e], 0), m_rows);
      const int t = min(max(m_indptr[e + 1], s), m_rows);
      s_row0[e] = s;
      c += (t - s + 63) / 64;
    }
  }
  int incl = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  int run = incl - c;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) {
      s_t0[e] = run;
      const int s = s_row0[e];
      const int t = min(max(m_indptr[e + 1], s), m_rows);
      run += (t - s + 63) / 64;
    }
  }
  if (lane == 63) {
    s_t0[E] = incl;
    s_row0[E] = min(max(m_indptr[E], 0), m_rows);
  }
}


// wait until at most N of this wavefront's loads are outstanding and its LDS
// reads have returned, then barrier
template <int N>
__device__ __forceinline__ void gd_wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));  // vmcnt(N) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}
constexpr int GD4_STAGE = 192 * 64;  // 64 + 128 rows of 128 bytes

// 64 x 128 tile, 8 wavefronts of 32 x 32, four LDS stages (each its own
// array): the loads of step kt+3 are issued at the start of step kt and
// waited for at the barrier that ends step kt+2 (vmcnt leaves the two later
// stages in flight); the fragment reads of a stage need no load wait.  The
// DMA mapping, swizzle and zero rows past the group are those of gd_tile.
// b is loaded with the streaming (non-temporal) cache policy: weights that
// come from memory (the usual case: other layers' weights pass through the
// caches between two calls) stream faster -- uniform E=8 x 128 rows, k=4096,
// n=2048: 67 -> 47 us -- but b is then not kept in the memory-side cache for
// the next call, so back-to-back calls on cached weights take 45 instead of
// 35 us.
template <bool F16, typename OutT>
__device__ __forceinline__ void gd4_tile(const uint16_t* __restrict__ a,
                                         const uint16_t* __restrict__ b, OutT* __restrict__ out,
                                         uint16_t* s0, uint16_t* s1, uint16_t* s2, uint16_t* s3,
                                         int e, int m0, int rows, int n0, int k, int n) {
  constexpr int WN = 4, BM = 64, BN = 128, R = BM + BN, NI = R / 64, NIA = BM / 64;  // 2 x 4 waves
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int r = lane & 31, h = lane >> 5;
  const int KT = k / GB_BK;
  const uint32_t kbytes = static_cast<uint32_t>(k) * 2;
  const __amdgpu_buffer_rsrc_t br =
      buf_rsrc(b + (static_cast<long>(e) * n + n0) * k, static_cast<uint32_t>(BN) * kbytes);
  const int lr = lane >> 3, lc = lane & 7;
  const uint32_t dvo = static_cast<uint32_t>(lr) * kbytes + ((lc ^ lr ^ (wave & 3)) << 4);
  __amdgpu_buffer_rsrc_t ari[NIA];
#pragma unroll
  for (int i = 0; i < NIA; ++i) {
    const int r0 = 8 * (8 * i + wave);
    ari[i] = buf_rsrc(a + static_cast<long>(m0 + r0) * k,
                      static_cast<uint32_t>(max(rows - r0, 0)) * kbytes);
  }
  auto dma = [&](uint16_t* st, int kt) {
    const uint32_t so = static_cast<uint32_t>(min(kt, KT - 1)) * (GB_BK * 2);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int g = 8 * i + wave;
      uint16_t* dst = st + g * 512;
      if (i < NIA)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ari[i], lds_ptr(dst), 16, dvo, so, 0, 0);
      else  // b: streaming (non-temporal) loads
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            br, lds_ptr(dst), 16, dvo, so + static_cast<uint32_t>(8 * g - BM) * kbytes, 0, 2);
    }
  };
  int fo[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) fo[s] = r * 64 + (((2 * s + h) ^ gd_swz(r)) << 3);
  f32x16 acc;
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[q] = 0.f;
  auto kstep = [&](int kt, const uint16_t* cur, uint16_t* nx3) {
    dma(nx3, kt + 3);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 fa = *reinterpret_cast<const u32x4*>(cur + wm * 32 * 64 + fo[s]);
      const u32x4 fb = *reinterpret_cast<const u32x4*>(cur + (BM / 32 + wn) * 32 * 64 + fo[s]);
      acc = mfma32<F16>(fb, fa, acc);
    }
    gd_wait_barrier<2 * NI>();
  };
  dma(s0, 0);
  dma(s1, 1);
  dma(s2, 2);
  gd_wait_barrier<2 * NI>();
  int kt = 0;
  for (; kt + 4 <= KT; kt += 4) {
    kstep(kt, s0, s3);
    kstep(kt + 1, s1, s0);
    kstep(kt + 2, s2, s1);
    kstep(kt + 3, s3, s2);
  }
  if (kt < KT) kstep(kt++, s0, s3);
  if (kt < KT) kstep(kt++, s1, s0);
  if (kt < KT) kstep(kt++, s2, s1);
  __builtin_amdgcn_s_waitcnt(0x0070);
  if (wm * 32 >= rows) return;
  const __amdgpu_buffer_rsrc_t orsrc = buf_rsrc(out + static_cast<long>(m0) * n,
                                                static_cast<uint32_t>(rows) * n * sizeof(OutT));
  const uint32_t orow = (static_cast<uint32_t>(wm * 32 + r) * n + n0 + wn * 32 + 4 * h) * sizeof(OutT);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 v = {acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
    bstore_out4<OutT>(orsrc, orow + 8 * g * sizeof(OutT), v);
  }
}

template <bool F16, typename OutT>
__global__ __launch_bounds__(64 * GD_WAVES, 1) void grouped_mm_dma64_kernel(
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
    const int32_t* __restrict__ m_indptr, OutT* __restrict__ out, int m_rows, int k, int n,
    int E) {
  __shared__ __attribute__((aligned(16))) uint16_t s0[GD4_STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t s1[GD4_STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t s2[GD4_STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t s3[GD4_STAGE];
  // the walk's tables live in the last stage, which the first K step's loads
  // overwrite only after the barrier that follows the first three stages
  static_assert(2 * (GM_MAX_EXPERTS + 1) * sizeof(int) <= GD4_STAGE * sizeof(uint16_t), "tables");
  int* const s_t0 = reinterpret_cast<int*>(s3);
  int* const s_row0 = s_t0 + (GM_MAX_EXPERTS + 1);
  if ((threadIdx.x >> 6) == 0) gd64_walk(m_indptr, m_rows, E, s_t0, s_row0);
  __syncthreads();
  const int nt = n / 128;
  const int count = s_t0[E];
  const long total = static_cast<long>(count) * nt;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const long run = (total + 7) / 8;
  const long L = xcd * run + slot;
  if (slot >= run || L >= total) return;
  int mt, ni;
  gb_order(L, count, nt, mt, ni);
  const int e = __builtin_amdgcn_readfirstlane(gb_owner(s_t0, E, mt));
  const int m0 = __builtin_amdgcn_readfirstlane(s_row0[e] + (mt - s_t0[e]) * 64);
  const int end = max(s_row0[e + 1], s_row0[e]);
  const int rows = __builtin_amdgcn_readfirstlane(min(end - m0, 64));
  gd4_tile<F16, OutT>(a, b, out, s0, s1, s2, s3, e, m0, rows, ni * 128, k, n);
}

template <bool F16, typename OutT>
mi_status launch_grouped_dma64(const void* a, int64_t m_rows, int64_t k, const void* b,
                               int64_t batch, int64_t n, const int32_t* m_indptr, void* out,
                               hipStream_t stream) {
  const long ub_tiles = ((m_rows + 63) / 64 + batch) * (n / 128);
  const long G = ((ub_tiles + 7) / 8 + 2) * 8;
  MI_REQUIRE(G < (1L << 31), "grouped_mm_bf16: problem too large");
  hipLaunchKernelGGL((grouped_mm_dma64_kernel<F16, OutT>), dim3(G), dim3(64 * GD_WAVES), 0,
                     stream, static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b),
                     m_indptr, static_cast<OutT*>(out), static_cast<int>(m_rows),
                     static_cast<int>(k), static_cast<int>(n), static_cast<int>(batch));
  return launch_status("grouped_mm_bf16");
}

template <bool F16, bool GLU, typename OutT>
__global__ __launch_bounds__(256, 1) void grouped_mm_big_kernel(
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
    const int32_t* __restrict__ m_indptr, OutT* __restrict__ out, int m_rows, int k, int n,
    int E, GbGlu gl) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * GB_STAGE];
  __shared__ int s_full0[GM_MAX_EXPERTS + 1];
  __shared__ int s_half0[GM_MAX_EXPERTS + 1];
  __shared__ int s_row0[GM_MAX_EXPERTS + 1];

  if ((threadIdx.x >> 6) == 0) gb_walk(m_indptr, m_rows, E, s_full0, s_half0, s_row0);
  __syncthreads();

  const int nt = n / GB_BN;
  const int count_f = s_full0[E], count_h = s_half0[E];
  const long total_f = static_cast<long>(count_f) * nt, total_h = static_cast<long>(count_h) * nt;
  // The grid is an upper bound on the tiles; the dispatcher deals workgroup
  // ids to the 8 XCDs in turn.  An XCD's first run_f workgroups take its run
  // of the 256-row tiles, the next run_h its run of the 128-row tiles.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const long run_f = (total_f + 7) / 8, run_h = (total_h + 7) / 8;
  if (slot < run_f) {
    const long L = xcd * run_f + slot;
    if (L >= total_f) return;
    int mt, ni;
    gb_order(L, count_f, nt, mt, ni);
    const int e = __builtin_amdgcn_readfirstlane(gb_owner(s_full0, E, mt));
    const int m0 = __builtin_amdgcn_readfirstlane(s_row0[e] + (mt - s_full0[e]) * 256);
    const int end = max(s_row0[e + 1], s_row0[e]);
    const int rows = __builtin_amdgcn_readfirstlane(min(end - m0, 256));
    gb_tile<4, GB_P, F16, GLU, OutT>(a, b, out, smem, e, m0, rows, ni * GB_BN, k, n, gl);
  } else {
    const long L = xcd * run_h + (slot - run_f);
    if (slot - run_f >= run_h || L >= total_h) return;
    int mt, ni;
    gb_order(L, count_h, nt, mt, ni);
    const int e = __builtin_amdgcn_readfirstlane(gb_owner(s_half0, E, mt));
    // the expert's last piece: after its 256-row tiles
    const int m0 = __builtin_amdgcn_readfirstlane(s_row0[e] + (s_full0[e + 1] - s_full0[e]) * 256);
    const int end = max(s_row0[e + 1], s_row0[e]);
    const int rows = __builtin_amdgcn_readfirstlane(end - m0);
    gb_tile<2, GB_PH, F16, GLU, OutT>(a, b, out, smem, e, m0, rows, ni * GB_BN, k, n, gl);
  }
}

template <bool F16, bool GLU, typename OutT>
mi_status launch_grouped_big(const void* a, int64_t m_rows, int64_t k, const void* b, int64_t batch,
                             int64_t n, const int32_t* m_indptr, void* out, hipStream_t stream,
                             const GbGlu& gl) {
  // one workgroup per tile of the upper bound (the real count is known on the
  // device only); each XCD's run of the real tiles fits in its G/8 ids
  const long ub_tiles = ((m_rows + 255) / 256 + batch) * (n / GB_BN);
  const long G = ((ub_tiles + 7) / 8 + 2) * 8;
  MI_REQUIRE(G < (1L << 31), "grouped_mm_bf16: problem too large");
  MI_REQUIRE(static_cast<uint64_t>(k) * 2 * (GLU ? n / 2 + 128 : GB_BN) < (1ULL << 32) &&
                 static_cast<uint64_t>(n) * 256 * sizeof(OutT) < (1ULL << 32),
             "grouped_mm_bf16: n or k too large for 256-row tiles");
  hipLaunchKernelGGL((grouped_mm_big_kernel<F16, GLU, OutT>), dim3(G), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b), m_indptr,
                     static_cast<OutT*>(out), static_cast<int>(m_rows), static_cast<int>(k),
                     static_cast<int>(n), static_cast<int>(batch), gl);
  return launch_status(GLU ? "grouped_mm_swiglu" : "grouped_mm_bf16");
}

template <bool F16, bool GLU, typename OutT>
mi_status launch_grouped_dma(const void* a, int64_t m_rows, int64_t k, const void* b,
                             int64_t batch, int64_t n, const int32_t* m_indptr, void* out,
                             hipStream_t stream, const GbGlu& gl) {
  // upper bound on the tiles of the three kinds: every tile covers at least
  // 128 rows of one expert or is its one partial tile, and at least 256
  // columns' worth of n-panels
  const long ub_tiles = ((m_rows + 127) / 128 + batch) * (n / 256);
  const long G = ((ub_tiles + 7) / 8 + 4) * 8;
  MI_REQUIRE(G < (1L << 31), "grouped_mm_bf16: problem too large");
  hipLaunchKernelGGL((grouped_mm_dma_kernel<F16, GLU, OutT>), dim3(G), dim3(64 * GD_WAVES), 0,
                     stream, static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b),
                     m_indptr, static_cast<OutT*>(out), static_cast<int>(m_rows),
                     static_cast<int>(k), static_cast<int>(n), static_cast<int>(batch), gl);
  return launch_status(GLU ? "grouped_mm_swiglu" : "grouped_mm_bf16");
}

template <bool F16, typename OutT>
mi_status dispatch_grouped(const void* a, int64_t m_rows, int64_t k, const void* b,
                           int64_t batch, int64_t n, const int32_t* m_indptr, void* out,
                           hipStream_t stream) {
  // Tile shape from host-known sizes only (the counts live on the device):
  // large average groups take 384x256 / 256x256 / 128x512 tiles (n % 512 ==
  // 0) or 256x256 tiles; smaller groups stream b from HBM and take 64x128
  // tiles.  k < 2^22 (checked by the caller) keeps every b panel's byte range
  // inside one buffer descriptor.
  const int64_t avg = m_rows / batch;
  if (avg >= 192 && n % 512 == 0 && static_cast<uint64_t>(n) * 384 * sizeof(OutT) < (1ULL << 32))
    return launch_grouped_dma<F16, false, OutT>(a, m_rows, k, b, batch, n, m_indptr, out, stream,
                                                GbGlu{});
  if (avg >= 192)
    return launch_grouped_big<F16, false, OutT>(a, m_rows, k, b, batch, n, m_indptr, out, stream,
                                               GbGlu{});
  return launch_grouped_dma64<F16, OutT>(a, m_rows, k, b, batch, n, m_indptr, out, stream);
}

}  // namespace
}  // namespace mi

extern "C" mi_status mi_grouped_mm_bf16(const void* a, int64_t m_rows, int64_t k, mi_dtype ab_dtype,
                                        const void* b, int64_t batch, int64_t n,
                                        const int32_t* m_indptr, void* out, mi_dtype out_dtype,
                                        void* stream) {
  using namespace mi;
  clear_error();
  MI_REQUIRE(batch >= 1, "grouped_mm_bf16: batch_size must be >= 1 (got %lld)", (long long)batch);
  MI_REQUIRE(batch <= GM_MAX_EXPERTS, "grouped_mm_bf16: batch_size must be <= %d (got %lld)",
             GM_MAX_EXPERTS, (long long)batch);
  MI_REQUIRE(m_rows >= 0 && m_rows < (1LL << 31), "grouped_mm_bf16: cum_m out of range (%lld)",
             (long long)m_rows);
  MI_REQUIRE(n > 0 && n % 256 == 0, "grouped_mm_bf16: n %% 256 == 0 required (got n=%lld)",
             (long long)n);
  MI_REQUIRE(k > 0 && k % 64 == 0, "grouped_mm_bf16: k %% 64 == 0 required (got k=%lld)",
             (long long)k);
  MI_REQUIRE(n < (1LL << 31) && k < (1LL << 31), "grouped_mm_bf16: n or k too large");
  MI_REQUIRE_SUPPORTED(k < (1LL << 22),
                       "grouped_mm_bf16: k < 4194304 required (a 512-row panel of b must fit one "
                       "32-bit buffer range; got k=%lld)", (long long)k);
  MI_REQUIRE(ab_dtype == MI_BF16 || ab_dtype == MI_F16,
             "grouped_mm_bf16: a and b must be bf16 or fp16");
  MI_REQUIRE(out_dtype == MI_BF16 || out_dtype == MI_F32 || out_dtype == MI_F16,
             "grouped_mm_bf16: out_dtype must be bf16, fp16 or fp32");
  MI_REQUIRE(m_indptr != nullptr, "grouped_mm_bf16: m_indptr is null");
  MI_REQUIRE(b != nullptr, "grouped_mm_bf16: b is null");
  if (m_rows == 0) return MI_OK;
  MI_REQUIRE(a != nullptr && out != nullptr, "grouped_mm_bf16: a/out is null");
  MI_REQUIRE(aligned16(a) && aligned16(b), "grouped_mm_bf16: a and b must be 16-byte aligned");
  MI_REQUIRE(aligned16(out), "grouped_mm_bf16: out must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool f16 = ab_dtype == MI_F16;
  if (out_dtype == MI_BF16)
    return f16 ? dispatch_grouped<true, Bf16Out>(a, m_rows, k, b, batch, n, m_indptr, out, s)
               : dispatch_grouped<false, Bf16Out>(a, m_rows, k, b, batch, n, m_indptr, out, s);
  if (out_dtype == MI_F16)
    return f16 ? dispatch_grouped<true, _Float16>(a, m_rows, k, b, batch, n, m_indptr, out, s)
               : dispatch_grouped<false, _Float16>(a, m_rows, k, b, batch, n, m_indptr, out, s);
  return f16 ? dispatch_grouped<true, float>(a, m_rows, k, b, batch, n, m_indptr, out, s)
             : dispatch_grouped<false, float>(a, m_rows, k, b, batch, n, m_indptr, out, s);
}

extern "C" mi_status mi_grouped_mm_swiglu(const void* a, int64_t m_rows, int64_t k,
                                          mi_dtype ab_dtype, const void* b, int64_t batch,
                                          int64_t inter_size, const int32_t* m_indptr,
                                          const void* fc1_delta, const float* alpha,
                                          const float* beta, const float* limit, void* out,
                                          mi_dtype out_dtype, void* stream) {
  using namespace mi;
  clear_error();
  MI_REQUIRE(batch >= 1 && batch <= GM_MAX_EXPERTS,
             "grouped_mm_swiglu: batch_size must be in [1, %d] (got %lld)", GM_MAX_EXPERTS,
             (long long)batch);
  MI_REQUIRE(m_rows >= 0 && m_rows < (1LL << 31), "grouped_mm_swiglu: cum_m out of range");
  MI_REQUIRE(inter_size > 0 && inter_size % 128 == 0 && inter_size < (1LL << 30),
             "grouped_mm_swiglu: intermediate size %% 128 == 0 required (got %lld)",
             (long long)inter_size);
  MI_REQUIRE(k > 0 && k % 64 == 0 && k < (1LL << 31),
             "grouped_mm_swiglu: k %% 64 == 0 required (got k=%lld)", (long long)k);
  MI_REQUIRE(ab_dtype == MI_BF16 || ab_dtype == MI_F16,
             "grouped_mm_swiglu: a and b must be bf16 or fp16");
  MI_REQUIRE(out_dtype == MI_BF16 || out_dtype == MI_F32 || out_dtype == MI_F16,
             "grouped_mm_swiglu: out_dtype must be bf16, fp16 or fp32");
  MI_REQUIRE(m_indptr != nullptr && b != nullptr, "grouped_mm_swiglu: m_indptr or b is null");
  if (m_rows == 0) return MI_OK;
  MI_REQUIRE(a != nullptr && out != nullptr, "grouped_mm_swiglu: a/out is null");
  MI_REQUIRE(aligned16(a) && aligned16(b), "grouped_mm_swiglu: a and b must be 16-byte aligned");
  MI_REQUIRE(fc1_delta == nullptr || (reinterpret_cast<uintptr_t>(fc1_delta) & 7) == 0,
             "grouped_mm_swiglu: fc1_delta must be 8-byte aligned");
  MI_REQUIRE((reinterpret_cast<uintptr_t>(out) & 15) == 0,
             "grouped_mm_swiglu: out must be 16-byte aligned");
  const int64_t n = 2 * inter_size;
  const GbGlu gl{static_cast<const uint16_t*>(fc1_delta), alpha, beta, limit};
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool f16 = ab_dtype == MI_F16;
  // large average groups with 512-wide panels (I % 256 == 0) take the
  // direct-to-LDS tiles, the rest the register-staged 256 x 256 ones
  const size_t osz = out_dtype == MI_F32 ? 4 : 2;
  const bool dma = m_rows / batch >= 192 && n % 512 == 0 &&
                   static_cast<uint64_t>(k) * 2 * 512 < (1ULL << 32) &&
                   static_cast<uint64_t>(k) * 2 * (inter_size + 256) < (1ULL << 32) &&
                   static_cast<uint64_t>(inter_size) * 384 * osz < (1ULL << 32);
#define MI_SWIGLU_LAUNCH(F16_, OutT_)                                                          \
  return dma ? launch_grouped_dma<F16_, true, OutT_>(a, m_rows, k, b, batch, n, m_indptr, out, s, \
                                                     gl)                                         \
             : launch_grouped_big<F16_, true, OutT_>(a, m_rows, k, b, batch, n, m_indptr, out, s, gl)
  if (out_dtype == MI_BF16) {
    if (f16) MI_SWIGLU_LAUNCH(true, Bf16Out);
    MI_SWIGLU_LAUNCH(false, Bf16Out);
  }
  if (out_dtype == MI_F16) {
    if (f16) MI_SWIGLU_LAUNCH(true, _Float16);
    MI_SWIGLU_LAUNCH(false, _Float16);
  }
  if (f16) MI_SWIGLU_LAUNCH(true, float);
  MI_SWIGLU_LAUNCH(false, float);
#undef MI_SWIGLU_LAUNCH
}
