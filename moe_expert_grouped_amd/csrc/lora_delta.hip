// FC2 LoRA delta of a routed MoE on gfx950.
//
// delta[t] = scale * sum_j w[t,j] * B_down[l,e] @ (A_down[l,e] @ act[perm[t*top_k+j]])
// (flashinfer.fused_moe.bgmv_moe_gemm2_lora_delta, formula and parameters).
//
// Work is organised around token tiles: up to TT tokens of one adapter.
// Four launches on the caller's stream, no host reads:
//
//  1. plan    (one workgroup) -- buckets the T tokens by adapter (bucket
//             num_adapters collects tokens without a valid adapter) and cuts
//             every bucket into tiles of <= TT tokens.
//  2. list    (one workgroup per tile) -- lists the tile's active slots
//             (permuted row in [0, padded_rows), expert in [0, num_experts))
//             by expert, each expert's list sorted by slot, and cuts every
//             list into 16-slot blocks.  Per block it stores the A_le and
//             B_le addresses and, per slot, the token row, activation row and
//             scale*w -- the block table both later kernels read.
//  3. shrink  (one wavefront per block) -- u = (scale*w) * A_le @ act[row]
//             with v_mfma_f32_16x16x32_bf16: the block's activation rows and
//             A_le are streamed with coalesced 16-byte loads (two K stages in
//             flight in registers) into a wave-private, swizzled LDS stage
//             and read back as MFMA fragments.  u is written as bf16 hi =
//             bf16(u) and lo = bf16(u - hi) (~16 significand bits together)
//             in the fragment order the expand consumes: one contiguous 1 KiB
//             record per block and 16 ranks; record i belongs to block i.
//             With fp16 activations and weights (lora_dtype fp16) the MFMAs
//             take fp16 and u, scaled per slot by a power of two, is carried
//             as fp16 hi + lo (details at the kernel).
//             When A_le fits in LDS (rank <= 32, 16 * ceil(rank/16) * I <=
//             32768, I % 128 == 0) the shrink runs per (adapter, expert)
//             instead: A_le is read once into LDS and the workgroup's
//             wavefronts take that pair's blocks from all of the adapter's
//             tiles (same records, same summation order).
//  4. expand  -- one workgroup per (tile, 128 output columns), in an order
//             that keeps the tiles of one column chunk on one XCD (they share
//             B columns through its L2).  An fp32 accumulator [TT tokens x 128
//             columns] lives in LDS.  Each of 4 wavefronts owns 32 columns and
//             walks the block table in order; per block it issues, for each of
//             its two 16-column groups, v_mfma_f32_16x16x32_bf16 on [B_le |
//             B_le] (16 columns x 32) and [u_hi ; u_lo] (32 x 16 slots) and
//             adds the 4 consecutive columns each lane holds into the slot's
//             token row with one 16-byte LDS read-modify-write.  The u record,
//             the B_le fragments (16 columns x 4 ranks per lane, 512 contiguous
//             bytes per wave) and the token rows of a block are loaded several
//             blocks ahead in a register ring.  The wavefront owns its columns
//             and a block never holds one token twice (unless the routing
//             repeats an expert for a token; such a tile uses LDS float
//             atomics), so every accumulator element is updated by one
//             wavefront in block order: the summation order per token is fixed
//             and the result is bitwise repeatable.  Tokens without adapter
//             get +0 rows.
#include <mutex>

#include "common.hpp"

// Scratch of the allocation-free delta entry point: one fixed array per GPU
// (each device the library runs on holds its own copy until the process
// ends).  Host code never passes this name to a kernel; it uses the device
// address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[MI_DELTA_SCRATCH_BYTES];

namespace mi {
namespace {

constexpr int PLAN_THREADS = 1024;
constexpr int MAX_ADAPTERS = 1023;  // + 1 "none" bucket
constexpr int MAX_TOPK = 32;
constexpr int MAX_EXPERTS = 512;
constexpr int SLOT_BUDGET = 1024;   // slots per tile (TT * top_k)
constexpr int NT_DELTA = 256;       // threads of the shrink and expand workgroups

struct Tile {
  int bucket, start, count, pad;
};

__device__ __forceinline__ Tile load_tile(const Tile* t) {
  return __builtin_bit_cast(Tile, gld<u32x4>(t));
}
__device__ __forceinline__ void store_tile(Tile* t, const Tile& v) {
  gst<u32x4>(t, __builtin_bit_cast(u32x4, v));
}

struct Layout {
  size_t u2, tok_list, tiles, counters, blk_a, blk_b, blk_tl, blk_row, blk_w, blk_f, tinfo,
      btile, tex, total;
  long cap;     // padded slot positions per tile
  int maxblk;   // 16-slot blocks per tile, at most
};

__host__ __device__ inline size_t al256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int tile_tokens(int64_t top_k) {
  int tt = 128;
  while (tt * top_k > SLOT_BUDGET) tt >>= 1;
  return tt;
}

int64_t max_tiles(int64_t T, int64_t top_k, int64_t L) { return T / tile_tokens(top_k) + L + 2; }

// every expert's list is padded to whole 16-slot blocks
long tile_capacity(int64_t top_k, int64_t E) {
  const long slots = static_cast<long>(tile_tokens(top_k)) * top_k;
  return slots + 15 * (E < slots ? E : slots);
}

// 16-rank chunks per slot, rounded up to 1, 2, 4 or 8
int rank_chunks(int64_t rank) {
  const int c = static_cast<int>((rank + 15) / 16);
  return c <= 1 ? 1 : c <= 2 ? 2 : c <= 4 ? 4 : 8;
}

Layout layout(int64_t T, int64_t top_k, int64_t E, int64_t L, int64_t rank) {
  Layout ly{};
  ly.cap = tile_capacity(top_k, E);
  const long nb = rank_chunks(rank);
  size_t off = 0;
  ly.u2 = off;
  off = al256(off + static_cast<size_t>(max_tiles(T, top_k, L)) * ly.cap * nb * 64);
  ly.tok_list = off;
  off = al256(off + static_cast<size_t>(T) * 4);
  ly.tiles = off;
  off = al256(off + static_cast<size_t>(max_tiles(T, top_k, L)) * sizeof(Tile));
  ly.counters = off;
  off = al256(off + 64);
  const size_t mt = static_cast<size_t>(max_tiles(T, top_k, L));
  ly.maxblk = static_cast<int>(ly.cap / 16 + 1);
  ly.blk_a = off;  // address of each block's A_le
  off = al256(off + mt * ly.maxblk * 8);
  ly.blk_b = off;  // address of each block's B_le
  off = al256(off + mt * ly.maxblk * 8);
  ly.blk_row = off;  // activation row of each slot (a valid row when the slot is empty)
  off = al256(off + mt * ly.maxblk * 64);
  ly.blk_w = off;  // scale * w of each slot (0 when empty)
  off = al256(off + mt * ly.maxblk * 64);
  ly.blk_f = off;  // fp16 carrier: power-of-two factor that undoes each slot's u scaling
  off = al256(off + mt * ly.maxblk * 64);
  ly.blk_tl = off;  // token row (tile-local) of each of a block's 16 slots, 0xFF = empty
  off = al256(off + mt * ly.maxblk * 16);
  ly.tinfo = off;  // per tile: number of blocks, "a token repeats an expert" flag
  off = al256(off + mt * 8);
  ly.btile = off;  // first tile of each adapter bucket (L + 2 entries)
  off = al256(off + static_cast<size_t>(L + 2) * 4);
  ly.tex = off;    // per tile: first block of each expert (E + 1 entries)
  off = al256(off + mt * static_cast<size_t>(E + 1) * 4);
  ly.total = off;
  return ly;
}

// ---------------------------------------------------------------------------
// 1. plan: tokens by adapter, tiles
// ---------------------------------------------------------------------------
struct PlanArgs {
  const int32_t* lora_ids;
  int T, L, tt;
  int32_t* tok_list;
  Tile* tiles;
  int32_t* counters;  // [0] = number of tiles
  int32_t* btile;     // [b] = first tile of bucket b, b = 0 .. L+1
};

__global__ __launch_bounds__(PLAN_THREADS) void plan_kernel(PlanArgs p) {
  __shared__ int s_cnt[MAX_ADAPTERS + 1];
  __shared__ int s_off[MAX_ADAPTERS + 1];
  __shared__ int s_tile0[MAX_ADAPTERS + 2];
  const int tid = threadIdx.x;
  const int nb = p.L + 1;
  for (int i = tid; i < nb; i += PLAN_THREADS) s_cnt[i] = 0;
  __syncthreads();
  for (int t = tid; t < p.T; t += PLAN_THREADS) {
    const int l = gld<int>(p.lora_ids + t);
    atomicAdd(&s_cnt[(l >= 0 && l < p.L) ? l : p.L], 1);
  }
  __syncthreads();
  if (tid < 64) {  // one wavefront scans the (<= 1024) buckets
    const int per = (nb + 63) / 64, b0 = tid * per;
    int tok = 0, til = 0;
    for (int i = 0; i < per; ++i)
      if (b0 + i < nb) {
        tok += s_cnt[b0 + i];
        til += (s_cnt[b0 + i] + p.tt - 1) / p.tt;
      }
    int itok = tok, itil = til;
    for (int o = 1; o < 64; o <<= 1) {
      const int a = __shfl_up(itok, o, 64), b = __shfl_up(itil, o, 64);
      if (tid >= o) {
        itok += a;
        itil += b;
      }
    }
    int rt = itok - tok, rl = itil - til;
    for (int i = 0; i < per; ++i)
      if (b0 + i < nb) {
        s_off[b0 + i] = rt;
        s_tile0[b0 + i] = rl;
        rt += s_cnt[b0 + i];
        rl += (s_cnt[b0 + i] + p.tt - 1) / p.tt;
      }
    if (tid == 63) {
      s_tile0[nb] = itil;
      gst<int>(p.counters, itil);
    }
  }
  __syncthreads();
  for (int b = tid; b <= nb; b += PLAN_THREADS) gst<int>(p.btile + b, s_tile0[b]);
  for (int b = tid; b < nb; b += PLAN_THREADS) {
    const int c = s_cnt[b];
    for (int i = 0; i * p.tt < c; ++i)
      store_tile(p.tiles + s_tile0[b] + i, Tile{b, s_off[b] + i * p.tt, min(p.tt, c - i * p.tt), 0});
  }
  __syncthreads();
  for (int t = tid; t < p.T; t += PLAN_THREADS) {
    const int l = gld<int>(p.lora_ids + t);
    gst<int>(p.tok_list + atomicAdd(&s_off[(l >= 0 && l < p.L) ? l : p.L], 1), t);
  }
}

// ---------------------------------------------------------------------------
// the tile's active slots, by expert (shared by shrink and expand)
// ---------------------------------------------------------------------------
struct SlotSrc {
  const int32_t* tok_list;
  const int32_t* perm;
  const int32_t* topk_ids;
  const float* topk_weights;
  int top_k, padded_rows, E;
};

struct SlotLists {
  int cnt[MAX_EXPERTS];       // scratch: counts, then write cursors
  int off[MAX_EXPERTS + 1];   // start of each expert in `list`
  int poff[MAX_EXPERTS + 1];  // start in the padded (whole-block) position space
  int list[SLOT_BUDGET];      // entries (t_local << 24 | x), ascending per expert
  int row[SLOT_BUDGET];       // permuted activation row of each entry
  float wgt[SLOT_BUDGET];     // routing weight of each entry
  int tmp[SLOT_BUDGET];       // scratch: unsorted entries
};

// All NT_DELTA threads call it.  Loads every slot of the tile once (two
// dependent rounds of loads), counts per expert, scans, scatters, and sorts
// each expert's list (one thread per expert) so that the order is the same
// in every workgroup that lists this tile.
__device__ void list_slots(const SlotSrc& s, const Tile& tile, SlotLists& L) {
  constexpr int PER = SLOT_BUDGET / NT_DELTA;
  const int tid = threadIdx.x;
  const int nslots = tile.count * s.top_k;
  int xs[PER], es[PER], rs[PER];
  float ws[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = tid + k * NT_DELTA;
    xs[k] = -1;
    if (i < nslots) {
      const int tl = i / s.top_k;
      xs[k] = gld<int>(s.tok_list + tile.start + tl) * s.top_k + (i - tl * s.top_k);
    }
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    es[k] = -1;
    rs[k] = 0;
    ws[k] = 0.f;
    if (xs[k] >= 0) {
      const int e = gld<int>(s.topk_ids + xs[k]), r = gld<int>(s.perm + xs[k]);
      ws[k] = s.topk_weights ? gld<float>(s.topk_weights + xs[k]) : 1.f;  // FC1: no weight
      if (e >= 0 && e < s.E && r >= 0 && r < s.padded_rows) es[k] = e;
      rs[k] = r;
    }
  }
  for (int i = tid; i < s.E; i += NT_DELTA) L.cnt[i] = 0;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < PER; ++k)
    if (es[k] >= 0) atomicAdd(&L.cnt[es[k]], 1);
  __syncthreads();
  if (tid < 64) {
    const int per = (s.E + 63) / 64, b0 = tid * per;
    int loc = 0, ploc = 0;
    for (int i = 0; i < per; ++i)
      if (b0 + i < s.E) {
        loc += L.cnt[b0 + i];
        ploc += (L.cnt[b0 + i] + 15) & ~15;
      }
    int inc = loc, pinc = ploc;
    for (int o = 1; o < 64; o <<= 1) {
      const int a = __shfl_up(inc, o, 64), b = __shfl_up(pinc, o, 64);
      if (tid >= o) {
        inc += a;
        pinc += b;
      }
    }
    int run = inc - loc, prun = pinc - ploc;
    for (int i = 0; i < per; ++i)
      if (b0 + i < s.E) {
        const int c = L.cnt[b0 + i];
        L.off[b0 + i] = run;
        L.poff[b0 + i] = prun;
        L.cnt[b0 + i] = run;  // write cursor
        run += c;
        prun += (c + 15) & ~15;
      }
    if (tid == 63) {
      L.off[s.E] = inc;
      L.poff[s.E] = pinc;
    }
  }
  __syncthreads();
  int pos[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    pos[k] = -1;
    if (es[k] >= 0) {
      const uint32_t tl = static_cast<uint32_t>((tid + k * NT_DELTA) / s.top_k);
      xs[k] = static_cast<int>((tl << 24) | static_cast<uint32_t>(xs[k]));  // the entry
      pos[k] = atomicAdd(&L.cnt[es[k]], 1);
      L.tmp[pos[k]] = xs[k];
    }
  }
  __syncthreads();
  // rank of each entry inside its expert's list (entries are distinct)
#pragma unroll
  for (int k = 0; k < PER; ++k)
    if (pos[k] >= 0) {
      const int b = L.off[es[k]], n = L.off[es[k] + 1] - b;
      const uint32_t v = static_cast<uint32_t>(xs[k]);
      int rank = 0;
      for (int i = 0; i < n; ++i) rank += static_cast<uint32_t>(L.tmp[b + i]) < v ? 1 : 0;
      L.list[b + rank] = xs[k];
      L.row[b + rank] = rs[k];
      L.wgt[b + rank] = ws[k];
    }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// 2. list: the tile's slots by expert, cut into 16-slot blocks (block table)
// ---------------------------------------------------------------------------
struct ListArgs {
  SlotSrc src;
  const Tile* tiles;
  const int32_t* counters;
  const float* topk_weights;
  const int64_t* w_ptr_a;
  long stride_a;
  const int64_t* w_ptr_b;
  long stride_b;
  int64_t* blk_a;     // per block: address of its A_le
  int64_t* blk_b;     // per block: address of its B_le
  uint32_t* blk_tl;   // per block: tile-local token row of each slot, 0xFF = empty
  int32_t* blk_row;   // per block: activation row of each slot (a valid row when empty)
  float* blk_w;       // per block: scale * w of each slot, 0 when empty
  int32_t* tinfo;     // per tile: number of blocks, "a token repeats an expert" flag
  int32_t* tex;       // per tile: first block of each expert, E + 1 entries
  int L, maxblk;
  float scale;
};

// One workgroup per tile.  Blocks are numbered in expert order (the u2
// record of block i is record i); every table entry a later kernel reads is
// written here, tiles without adapter included (zero blocks).
__global__ __launch_bounds__(NT_DELTA) void list_kernel(ListArgs p) {
  __shared__ SlotLists SL;
  __shared__ int64_t s_pa[MAX_EXPERTS], s_pb[MAX_EXPERTS];  // A_le, B_le of each expert
  const int ti = blockIdx.x;
  if (ti >= gld<int>(p.counters)) return;
  const Tile tile = load_tile(p.tiles + ti);
  if (tile.bucket >= p.L) {
    if (threadIdx.x == 0) gst<uint64_t>(p.tinfo + 2 * ti, 0ull);
    return;
  }
  const int l = tile.bucket;
  const int E = p.src.E;
  for (int e = threadIdx.x; e < E; e += NT_DELTA) {  // in flight with the slot loads
    s_pa[e] = gld<int64_t>(p.w_ptr_a + e) + 2 * p.stride_a * l;
    s_pb[e] = gld<int64_t>(p.w_ptr_b + e) + 2 * p.stride_b * l;
  }
  list_slots(p.src, tile, SL);  // starts and ends with barriers
  const long tb = static_cast<long>(ti) * p.maxblk;
  for (int e = threadIdx.x; e <= E; e += NT_DELTA)
    gst<int>(p.tex + static_cast<long>(ti) * (E + 1) + e, SL.poff[e] >> 4);

  // per block: its A_le and B_le (one thread per expert, ~1 block each)
  for (int e = threadIdx.x; e < E; e += NT_DELTA) {
    const int n = SL.off[e + 1] - SL.off[e];
    if (n == 0) continue;
    const int64_t ale = s_pa[e], ble = s_pb[e];
    for (int b = 0; b * 16 < n; ++b) {
      gst<int64_t>(p.blk_a + tb + (SL.poff[e] >> 4) + b, ale);
      gst<int64_t>(p.blk_b + tb + (SL.poff[e] >> 4) + b, ble);
    }
  }
  // per 4-slot word of the padded position space: token rows, act rows, weights
  const int npos = SL.poff[E];
  int dup = 0;
  for (int w = threadIdx.x; w < npos / 4; w += NT_DELTA) {
    const int p0 = 4 * w;
    int lo = 0, hi = E;  // the expert owning p0: last e with poff[e] <= p0
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (SL.poff[mid] <= p0) lo = mid; else hi = mid;
    }
    const int e = lo, b0 = SL.off[e], n = SL.off[e + 1] - b0, k0 = p0 - SL.poff[e];
    uint32_t tlw = 0;
    u32x4 rows, ws;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const int k = k0 + s2;
      const int entry = SL.list[b0 + min(k, n - 1)];  // empty slots repeat a valid row
      const uint32_t tl = static_cast<uint32_t>(entry) >> 24;
      tlw |= (k < n ? tl : 0xFFu) << (8 * s2);
      rows[s2] = static_cast<uint32_t>(SL.row[b0 + min(k, n - 1)]);
      ws[s2] = __float_as_uint(k < n ? p.scale * SL.wgt[b0 + k] : 0.f);
      if (k > 0 && k < n)  // the list is sorted by token: a repeat is adjacent
        dup |= (static_cast<uint32_t>(SL.list[b0 + k - 1]) >> 24) == tl;
    }
    gst<uint32_t>(p.blk_tl + tb * 4 + w, tlw);
    gst<u32x4>(p.blk_row + tb * 16 + p0, rows);
    gst<u32x4>(p.blk_w + tb * 16 + p0, ws);
  }
  dup = __syncthreads_or(dup);
  if (threadIdx.x == 0) {
    gst<int>(p.tinfo + 2 * ti, npos >> 4);
    gst<int>(p.tinfo + 2 * ti + 1, dup);
  }
}

// u2 record of one 16-slot block: NB chunks of 16 ranks, each 64 lane groups
// of 8 bf16 -- the expand's MFMA operand of lane (slot, q) = slot + 16 q,
// which holds hi then lo of ranks 4q .. 4q+3 of the chunk (part 0 hi, 1 lo).
__device__ __forceinline__ int u2_elem(int c, int part, int slot, int rr) {
  return c * 512 + ((rr >> 2) * 16 + slot) * 8 + part * 4 + (rr & 3);
}

// u of one block from the MFMA accumulators: acc[nb][j] = (A_le @ act)[slot
// 4kq + j][rank 16nb + row].  Scales by scale*w (bw: the block's 16 weights,
// 0 for empty slots), splits into hi + lo and writes the block's u record
// (F16: per-slot power-of-two scaling first, factors to bf).
template <int NB, bool F16>
__device__ __forceinline__ void shrink_store(const f32x4 (&acc)[NB], uint16_t* rec, const float* bw,
                                             float* bf, int rank) {
  const int lane = threadIdx.x & 63, row = lane & 15, kq = lane >> 4;
  // acc[nb][j] = (A_le @ act)[slot 4*kq + j][rank nb*16 + row]; empty slots have weight 0
  const f32x4 wv = __builtin_bit_cast(f32x4, gld<u32x4>(bw + 4 * kq));
  f32x4 fac = f32x4{1.f, 1.f, 1.f, 1.f};  // F16: 2^-k of each of the lane group's 4 slots
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int srow = 4 * kq + j;
    float v[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) v[nb] = nb * 16 + row < rank ? acc[nb][j] * wv[j] : 0.f;
    if constexpr (F16) {
      // slot maximum over the 16 lanes of this lane group (ranks row, row+16, ...)
      float m = 0.f;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) m = fmaxf(m, fabsf(v[nb]));
#pragma unroll
      for (int x = 1; x < 16; x <<= 1) m = fmaxf(m, __shfl_xor(m, x));
      // m in [2^(ex-1), 2^ex) -> m * 2^(15-ex) in [2^14, 2^15); the clamp keeps
      // 2^-k a normal float (a slot that small stays scaled up by 2^112)
      const int k = min(max(15 - __builtin_amdgcn_frexp_expf(m), -113), 112);
      fac[j] = __builtin_amdgcn_ldexpf(1.f, -k);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float us = __builtin_amdgcn_ldexpf(v[nb], k);
        const _Float16 hi = static_cast<_Float16>(us);
        const _Float16 lo = static_cast<_Float16>(us - static_cast<float>(hi));
        gst<uint16_t>(rec + u2_elem(nb, 0, srow, row), __builtin_bit_cast(uint16_t, hi));
        gst<uint16_t>(rec + u2_elem(nb, 1, srow, row), __builtin_bit_cast(uint16_t, lo));
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint32_t hi = f32_to_bf16_rne(v[nb]);
        const uint32_t lo = f32_to_bf16_rne(v[nb] - bf16_bits_to_f32(hi));
        gst<uint16_t>(rec + u2_elem(nb, 0, srow, row), static_cast<uint16_t>(hi));
        gst<uint16_t>(rec + u2_elem(nb, 1, srow, row), static_cast<uint16_t>(lo));
      }
    }
  }
  if (F16 && row == 0) gst<f32x4>(bf + 4 * kq, fac);
}

// ---------------------------------------------------------------------------
// 3. shrink: u = (scale * w) * A_le @ act[row], one wavefront per block
// ---------------------------------------------------------------------------
constexpr int SHR_WAVES = 4;  // wavefronts (blocks) per workgroup

struct ShrinkArgs {
  const uint16_t* act;
  const Tile* tiles;
  const int32_t* counters;
  const int64_t* blk_a;
  const int32_t* blk_row;
  const float* blk_w;
  const int32_t* tinfo;
  uint16_t* u2;
  float* blk_f;
  long cap;
  int I, L, rank, maxblk, bpt;  // bpt: workgroups per tile
};

// One 16x16x32 MFMA step of either input type (fp32 accumulation, exact products)
template <bool F16>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// The block's 16 activation rows and A_le are streamed with coalesced 16-byte
// loads (two K stages in flight in registers) into a wave-private, swizzled
// LDS stage and read back as v_mfma_f32_16x16x32_bf16 fragments.  (A fragment
// puts neighbouring lanes on different rows; loading it straight from memory
// costs more address work per byte.)  Waves never synchronise with each
// other, so a wave without a block just leaves.
//
// F16 (lora_dtype fp16): the MFMAs take fp16 and u is carried as fp16 hi + lo.
// fp16 has a narrow exponent range, so each slot's u row is first multiplied
// by 2^k, k chosen so that its largest magnitude lies in [2^14, 2^15); hi + lo
// then keep ~22 significant bits of every rank relative to that maximum and
// nothing overflows.  2^-k goes to blk_f and the expand multiplies it back
// (both scalings by powers of two are exact).
template <int NB, bool F16>  // NB: 1, 2, 4 or 8
__global__ __launch_bounds__(64 * SHR_WAVES) void shrink_kernel(ShrinkArgs p) {
  static_assert(NB == 1 || NB == 2 || NB == 4 || NB == 8, "rank chunks");
  constexpr int KC = (128 / NB) < 32 ? 32 : 128 / NB;  // K elements per LDS stage
  constexpr int CPR = KC / 8;                          // 16-byte chunks per stage row
  constexpr int RPI = 64 / CPR;                        // rows per coalesced load instruction
  constexpr int NLA = 16 / RPI;                        // act loads per lane per stage
  constexpr int NLB = 16 * NB / RPI;                   // A_le loads per lane per stage
  constexpr int STAGE = 16 * (1 + NB) * KC;            // bf16 per wave stage
  __shared__ __attribute__((aligned(16))) uint16_t s_stage[SHR_WAVES][STAGE];

  const int ti = blockIdx.x / p.bpt;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bi = (blockIdx.x % p.bpt) * SHR_WAVES + wave;
  if (ti >= gld<int>(p.counters)) return;
  if (load_tile(p.tiles + ti).bucket >= p.L) return;  // no adapter, no blocks
  if (bi >= gld<int>(p.tinfo + 2 * ti)) return;
  const long tb = static_cast<long>(ti) * p.maxblk + bi;

  const int row = lane & 15, kq = lane >> 4;      // MFMA fragment roles
  const int lrow = lane / CPR, lch = lane % CPR;  // coalesced-load roles
  uint16_t* stA = s_stage[wave];  // [16][KC]
  uint16_t* stB = stA + 16 * KC;  // [16*NB][KC]
  const uint16_t* Ale = reinterpret_cast<const uint16_t*>(gld<int64_t>(p.blk_a + tb));

  const uint16_t* asrc[NLA];
  const uint16_t* bsrc[NLB];
#pragma unroll
  for (int j = 0; j < NLA; ++j) {
    const int r = j * RPI + lrow;  // 0..15
    asrc[j] = p.act + static_cast<long>(gld<int>(p.blk_row + tb * 16 + r)) * p.I + lch * 8;
  }
#pragma unroll
  for (int j = 0; j < NLB; ++j) {
    const int r = j * RPI + lrow;  // rank row 0 .. 16*NB-1 (clamped to real ranks)
    bsrc[j] = Ale + static_cast<long>(min(r, p.rank - 1)) * p.I + lch * 8;
  }
  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nst = p.I / KC;  // full stages
  // two register stages in flight: stage st + 2 is loaded while st feeds the MFMAs
  u32x4 ra0[NLA], rb0[NLB], ra1[NLA], rb1[NLB];
  auto gload = [&](u32x4 (&ra)[NLA], u32x4 (&rb)[NLB], int st) {
    if (st < nst) {
      const int k0 = st * KC;
#pragma unroll
      for (int j = 0; j < NLA; ++j) ra[j] = gld_nt<u32x4>(asrc[j] + k0);  // rows read once
#pragma unroll
      for (int j = 0; j < NLB; ++j) rb[j] = gld<u32x4>(bsrc[j] + k0);
    }
  };
  auto consume = [&](u32x4 (&ra)[NLA], u32x4 (&rb)[NLB], int st) {
    // registers -> LDS; chunk c of stage row r sits at chunk c ^ (r % CPR)
#pragma unroll
    for (int j = 0; j < NLA; ++j) {
      const int r = j * RPI + lrow;
      *reinterpret_cast<u32x4*>(stA + r * KC + ((lch ^ (r % CPR)) << 3)) = ra[j];
    }
#pragma unroll
    for (int j = 0; j < NLB; ++j) {
      const int r = j * RPI + lrow;
      *reinterpret_cast<u32x4*>(stB + r * KC + ((lch ^ (r % CPR)) << 3)) = rb[j];
    }
    __builtin_amdgcn_wave_barrier();
    gload(ra, rb, st + 2);
#pragma unroll
    for (int s2 = 0; s2 < KC / 32; ++s2) {
      const int c = 4 * s2 + kq;
      const u32x4 fa =
          *reinterpret_cast<const u32x4*>(stA + row * KC + ((c ^ (row % CPR)) << 3));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int rr = nb * 16 + row;
        const u32x4 fb =
            *reinterpret_cast<const u32x4*>(stB + rr * KC + ((c ^ (rr % CPR)) << 3));
        acc[nb] = mfma16<F16>(fa, fb, acc[nb]);
      }
    }
    __builtin_amdgcn_wave_barrier();  // this stage's reads precede the next stage's writes
  };
  gload(ra0, rb0, 0);
  gload(ra1, rb1, 1);
  for (int st = 0; st < nst; st += 2) {
    consume(ra0, rb0, st);
    if (st + 1 < nst) consume(ra1, rb1, st + 1);
  }
  // K tail (I % KC != 0): fragments straight from memory
  for (int k0 = nst * KC; k0 < p.I; k0 += 32) {
    const bool kin = k0 + kq * 8 < p.I;  // I % 8 == 0
    const u32x4 fa =
        kin ? gld<u32x4>(p.act + static_cast<long>(gld<int>(p.blk_row + tb * 16 + row)) * p.I +
                         k0 + kq * 8)
            : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int rr = nb * 16 + row;
      const u32x4 fb = (kin && rr < p.rank)
                           ? gld<u32x4>(Ale + static_cast<long>(rr) * p.I + k0 + kq * 8)
                           : u32x4{0, 0, 0, 0};
      acc[nb] = mfma16<F16>(fa, fb, acc[nb]);
    }
  }
  shrink_store<NB, F16>(acc, p.u2 + (static_cast<long>(ti) * p.cap + bi * 16) * NB * 32,
                        p.blk_w + tb * 16, p.blk_f + tb * 16, p.rank);
}

// ---------------------------------------------------------------------------
// 3b. shrink by (adapter, expert): A_le read once into LDS
// ---------------------------------------------------------------------------
// The tiles of adapter l are consecutive and list each expert's blocks
// consecutively (tex), so the blocks that use one A_le are easy to enumerate.
// One workgroup per (l, e, part) keeps A_le in LDS (16*NB rows; used when they
// fit) and its 4 wavefronts take the blocks of (l, e) in the tiles
// btile[l] + part, + S, ... in turn; each streams its block's 16 activation
// rows through a wave-private stage as shrink_kernel does.  Per block this
// reads A_le from LDS instead of from the caches, which the per-tile shrink
// does once per block.
constexpr int SLE_KC = 128;          // activation K elements per wave stage
constexpr int SLE_SD = 6;            // activation stages in flight per wavefront
constexpr int SLE_AMAX = 16 * 2048;  // bf16 of A_le held in LDS: 16 * NB * I <= SLE_AMAX
constexpr int SLE_AMAX_BIG = 16 * 4096;  // the one-workgroup-per-CU variant (128 KB of A_le)

struct ShrinkLeArgs {
  const uint16_t* act;
  const int64_t* w_ptr_a;
  long stride_a;
  const int32_t* btile;
  const int32_t* tex;
  const int32_t* blk_row;
  const float* blk_w;
  uint16_t* u2;
  float* blk_f;
  long cap;
  int I, E, L, rank, maxblk, S;
};

template <int NB, bool F16, int AMAX>  // NB: 1 or 2; AMAX: bf16 of A_le the LDS holds
__global__ __launch_bounds__(256, AMAX > SLE_AMAX ? 1 : 2) void shrink_le_kernel(ShrinkLeArgs p) {
  constexpr int R16 = 16 * NB;       // A_le rows held (ranks past the rank repeat the last one)
  constexpr int CPR = SLE_KC / 8;    // 16-byte chunks per stage row
  constexpr int RPI = 64 / CPR;      // stage rows per coalesced load instruction
  constexpr int NLA = 16 / RPI;      // activation loads per lane per stage
  __shared__ __attribute__((aligned(16))) uint16_t s_a[AMAX];
  __shared__ __attribute__((aligned(16))) uint16_t s_act[4][16 * SLE_KC];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int le = blockIdx.x / p.S, part = blockIdx.x % p.S;
  const int l = le / p.E, e = le % p.E;
  if (l >= p.L) return;
  const int t0 = gld<int>(p.btile + l) + part, t1 = gld<int>(p.btile + l + 1);
  const int E1 = p.E + 1;
  int nblk = 0;  // blocks of (l, e) in this part's tiles (the same in every lane)
  for (int ti = t0; ti < t1; ti += p.S)
    nblk += gld<int>(p.tex + static_cast<long>(ti) * E1 + e + 1) -
            gld<int>(p.tex + static_cast<long>(ti) * E1 + e);
  if (nblk == 0) return;

  // A_le -> LDS: row r, 16-byte chunk c at chunk c ^ (r & 15) (I % 128 == 0)
  const int cpr = p.I / 8;
  const uint16_t* Ale =
      reinterpret_cast<const uint16_t*>(gld<int64_t>(p.w_ptr_a + e) + 2 * p.stride_a * l);
  // eight 16-byte loads per thread in flight before their LDS writes
  for (int c0 = 0; c0 < R16 * cpr; c0 += 8 * 256) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // past the end: reload the last chunk (not stored)
      const int c = min(c0 + u * 256 + tid, R16 * cpr - 1);
      const int r = c / cpr, cc = c - r * cpr;
      // streaming loads: each (adapter, expert) pair's A_le is read once, here
      v[u] = gld_nt<u32x4>(Ale + static_cast<long>(min(r, p.rank - 1)) * p.I + cc * 8);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = c0 + u * 256 + tid;
      const int r = c / cpr, cc = c - r * cpr;
      if (c < R16 * cpr) *reinterpret_cast<u32x4*>(s_a + r * p.I + ((cc ^ (r & 15)) << 3)) = v[u];
    }
  }
  __syncthreads();

  const int row = lane & 15, kq = lane >> 4;      // MFMA fragment roles
  const int lrow = lane / CPR, lch = lane % CPR;  // coalesced-load roles
  uint16_t* st = s_act[wave];
  const int nst = p.I / SLE_KC;  // I % 128 == 0
  int j = 0;
  for (int ti = t0; ti < t1; ti += p.S) {
    const int b0 = gld<int>(p.tex + static_cast<long>(ti) * E1 + e);
    const int b1 = gld<int>(p.tex + static_cast<long>(ti) * E1 + e + 1);
    for (int bi = b0; bi < b1; ++bi, ++j) {
      if ((j & 3) != wave) continue;
      const long tb = static_cast<long>(ti) * p.maxblk + bi;
      const uint16_t* asrc[NLA];
#pragma unroll
      for (int jj = 0; jj < NLA; ++jj) {
        const int r = jj * RPI + lrow;
        asrc[jj] = p.act + static_cast<long>(gld<int>(p.blk_row + tb * 16 + r)) * p.I + lch * 8;
      }
      f32x4 acc[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      // SLE_SD register stages in flight: stage s + SLE_SD is loaded while s
      // feeds the MFMAs
      u32x4 ra[SLE_SD][NLA];
      auto gload = [&](u32x4 (&r)[NLA], int s) {
        if (s < nst) {
#pragma unroll
          for (int jj = 0; jj < NLA; ++jj)  // activation rows are read once
            r[jj] = gld_nt<u32x4>(asrc[jj] + s * SLE_KC);
        }
      };
      auto consume = [&](u32x4 (&r)[NLA], int s) {
#pragma unroll
        for (int jj = 0; jj < NLA; ++jj) {
          const int rw = jj * RPI + lrow;
          *reinterpret_cast<u32x4*>(st + rw * SLE_KC + ((lch ^ (rw % CPR)) << 3)) = r[jj];
        }
        __builtin_amdgcn_wave_barrier();
        gload(r, s + SLE_SD);
#pragma unroll
        for (int s2 = 0; s2 < SLE_KC / 32; ++s2) {
          const int c = 4 * s2 + kq;
          const u32x4 fa =
              *reinterpret_cast<const u32x4*>(st + row * SLE_KC + ((c ^ (row % CPR)) << 3));
          const int ca = s * CPR + c;  // chunk of A_le's row
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int rr = nb * 16 + row;
            const u32x4 fb = *reinterpret_cast<const u32x4*>(s_a + rr * p.I + ((ca ^ (rr & 15)) << 3));
            acc[nb] = mfma16<F16>(fa, fb, acc[nb]);
          }
        }
        __builtin_amdgcn_wave_barrier();  // this stage's reads precede the next stage's writes
      };
#pragma unroll
      for (int q = 0; q < SLE_SD; ++q) gload(ra[q], q);
      for (int s = 0; s < nst; s += SLE_SD) {
#pragma unroll
        for (int q = 0; q < SLE_SD; ++q)
          if (s + q < nst) consume(ra[q], s + q);
      }
      shrink_store<NB, F16>(acc, p.u2 + (static_cast<long>(ti) * p.cap + bi * 16) * NB * 32,
                            p.blk_w + tb * 16, p.blk_f + tb * 16, p.rank);
    }
  }
}

// ---------------------------------------------------------------------------
// 4. expand
// ---------------------------------------------------------------------------
constexpr int EXP_CW = 128;   // output columns per workgroup
constexpr int NT_EXP = 256;   // expand workgroup: 4 wavefronts x 2 groups of 16 columns
constexpr int EXP_NCG = EXP_CW / 16 / (NT_EXP / 64);  // 16-column groups per wavefront
constexpr int EXP_TT = 128;   // accumulator rows (tokens per tile, at most)
constexpr int MAX_BLOCKS = SLOT_BUDGET / 16 + MAX_EXPERTS;
static_assert(EXP_CW == 16 * EXP_NCG * (NT_EXP / 64), "column groups");

struct ExpandArgs {
  const int32_t* tok_list;
  const Tile* tiles;
  const int32_t* counters;
  const uint16_t* u2;
  const int64_t* blk_b;
  const uint32_t* blk_tl;
  const float* blk_f;
  const int32_t* tinfo;
  void* out;
  long cap;
  int L, H, rank, maxblk, max_tiles, nch;
  int out_kind;  // 0 bf16, 1 fp32, 2 fp16
  // finalize (fc2 != NULL): add the routing-weighted FC2 rows of each token
  const void* fc2;
  const int32_t* perm;
  const float* topk_weights;
  int fc2_kind;  // 0 bf16, 1 fp32, 2 fp16
  int top_k, padded_rows;
};

// 8 consecutive values of an FC2 row as fp32 (exact conversions)
__device__ __forceinline__ void fc2_load8(const void* base, int kind, long off, f32x4& x0,
                                          f32x4& x1) {
  if (kind == 1) {
    x0 = gld<f32x4>(static_cast<const float*>(base) + off);
    x1 = gld<f32x4>(static_cast<const float*>(base) + off + 4);
  } else if (kind == 2) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const h8 h = __builtin_bit_cast(h8, gld<u32x4>(static_cast<const uint16_t*>(base) + off));
    x0 = f32x4{static_cast<float>(h[0]), static_cast<float>(h[1]), static_cast<float>(h[2]),
               static_cast<float>(h[3])};
    x1 = f32x4{static_cast<float>(h[4]), static_cast<float>(h[5]), static_cast<float>(h[6]),
               static_cast<float>(h[7])};
  } else {
    // streaming loads: each FC2 row piece is read once
    const u32x4 v = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + off));
    x0 = f32x4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
               __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u)};
    x1 = f32x4{__uint_as_float(v.z << 16), __uint_as_float(v.z & 0xFFFF0000u),
               __uint_as_float(v.w << 16), __uint_as_float(v.w & 0xFFFF0000u)};
  }
}

// 8 output columns of token t rounded once to the output type
__device__ __forceinline__ void store_out8(const ExpandArgs& p, int t, int col, f32x4 v0,
                                           f32x4 v1) {
  const long o = static_cast<long>(t) * p.H + col;
  if (p.out_kind == 1) {
    gst<f32x4>(static_cast<float*>(p.out) + o, v0);
    gst<f32x4>(static_cast<float*>(p.out) + o + 4, v1);
  } else if (p.out_kind == 2) {  // IEEE fp16, round to nearest even
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const h8 h = {static_cast<_Float16>(v0.x), static_cast<_Float16>(v0.y),
                  static_cast<_Float16>(v0.z), static_cast<_Float16>(v0.w),
                  static_cast<_Float16>(v1.x), static_cast<_Float16>(v1.y),
                  static_cast<_Float16>(v1.z), static_cast<_Float16>(v1.w)};
    gst<u32x4>(static_cast<uint16_t*>(p.out) + o, __builtin_bit_cast(u32x4, h));
  } else {
    u32x4 w;
    w.x = pack_bf16x2(v0.x, v0.y);
    w.y = pack_bf16x2(v0.z, v0.w);
    w.z = pack_bf16x2(v1.x, v1.y);
    w.w = pack_bf16x2(v1.z, v1.w);
    // streaming store: the output is not read again here
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.out) + o));
  }
}

// Finalize: the routed FC2 rows of a token, FIN_KB slots at a time.  A slot
// not routed here (row < 0 or >= padded_rows, or past top_k) gets row 0 and
// weight 0 and is skipped when summing.
constexpr int FIN_KB = 8;
struct Route {
  int r[FIN_KB];
  float w[FIN_KB];
};
__device__ __forceinline__ Route load_route(const ExpandArgs& p, int t, int j0) {
  Route rt;
#pragma unroll
  for (int jj = 0; jj < FIN_KB; ++jj) {
    const int j = j0 + jj;
    const long s = static_cast<long>(t) * p.top_k + j;
    const int rr = j < p.top_k ? gld<int>(p.perm + s) : -1;
    const bool ok = rr >= 0 && rr < p.padded_rows;
    rt.r[jj] = ok ? rr : 0;
    rt.w[jj] = ok ? gld<float>(p.topk_weights + s) : 0.f;
  }
  return rt;
}
struct Rows8 {
  f32x4 x0[FIN_KB], x1[FIN_KB];
};
__device__ __forceinline__ Rows8 load_rows(const ExpandArgs& p, const Route& rt, int col) {
  Rows8 x;
#pragma unroll
  for (int jj = 0; jj < FIN_KB; ++jj)
    fc2_load8(p.fc2, p.fc2_kind, static_cast<long>(rt.r[jj]) * p.H + col, x.x0[jj], x.x1[jj]);
  return x;
}
// v += sum over the batch of w * row, in slot order (one FMA each)
__device__ __forceinline__ void add_rows(const Route& rt, const Rows8& x, f32x4& v0, f32x4& v1) {
#pragma unroll
  for (int jj = 0; jj < FIN_KB; ++jj) {
    if (rt.w[jj] == 0.f) continue;  // not routed here (or a zero weight: adds nothing)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v0[q] = __builtin_fmaf(rt.w[jj], x.x0[jj][q], v0[q]);
      v1[q] = __builtin_fmaf(rt.w[jj], x.x1[jj][q], v1[q]);
    }
  }
}

// Write-out of a tile's TT x EXP_CW outputs, 8 columns per item, items tid,
// tid + NT_EXP, ...: the delta of item i comes from `delta(i)` (fp32), plus,
// when finalizing, the routed FC2 rows.  For top_k <= FIN_KB the loads are
// pipelined over items: the rows of item i and the routing of item i+NT_EXP
// are in flight together.
template <typename DeltaFn>
__device__ __forceinline__ void write_tile(const ExpandArgs& p, const Tile& tile, int h0,
                                           DeltaFn delta, const int* s_tok = nullptr) {
  const int tid = threadIdx.x;
  const int nit = tile.count * (EXP_CW / 8);
  // the tile's token ids, from LDS when the caller staged them there
  auto tok = [&](int i) {
    return s_tok ? s_tok[i / (EXP_CW / 8)] : gld<int>(p.tok_list + tile.start + i / (EXP_CW / 8));
  };
  auto colof = [&](int i) { return h0 + (i % (EXP_CW / 8)) * 8; };
  if (p.fc2 == nullptr) {
    for (int i = tid; i < nit; i += NT_EXP) {
      f32x4 v0, v1;
      delta(i, v0, v1);
      store_out8(p, tok(i), colof(i), v0, v1);
    }
    return;
  }
  if (p.top_k <= FIN_KB) {
    int t = tid < nit ? tok(tid) : 0;
    Route rt = load_route(p, tid < nit ? t : 0, tid < nit ? 0 : p.top_k);
    for (int i = tid; i < nit; i += NT_EXP) {
      const Rows8 x = load_rows(p, rt, colof(i));
      const int in = i + NT_EXP;
      const int tn = in < nit ? tok(in) : 0;
      const Route rn = load_route(p, tn, in < nit ? 0 : p.top_k);
      f32x4 v0, v1;
      delta(i, v0, v1);
      add_rows(rt, x, v0, v1);
      store_out8(p, t, colof(i), v0, v1);
      rt = rn;
      t = tn;
    }
    return;
  }
  for (int i = tid; i < nit; i += NT_EXP) {
    const int t = tok(i);
    f32x4 v0, v1;
    delta(i, v0, v1);
    for (int j0 = 0; j0 < p.top_k; j0 += FIN_KB) {
      const Route rt = load_route(p, t, j0);
      add_rows(rt, load_rows(p, rt, colof(i)), v0, v1);
    }
    store_out8(p, t, colof(i), v0, v1);
  }
}

// Finalize, second pass (when the workspace holds an fp32 [T, H] delta): one
// thread per 8 columns of one token reads the token's fp32 delta and its
// routed FC2 rows (whole rows across a wavefront, 16 or 32 bytes a lane) and
// writes the combined output.  The same arithmetic as write_tile's: the delta,
// then one FMA per routed slot in slot order, one rounding.
__global__ __launch_bounds__(256) void finalize_combine_kernel(ExpandArgs p, const float* delta,
                                                               int T) {
  const long cpr = p.H / 8;  // 8-column items per token
  const long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<long>(T) * cpr) return;
  const int t = static_cast<int>(i / cpr);
  const int col = static_cast<int>(i - t * cpr) * 8;
  const float* d = delta + static_cast<long>(t) * p.H + col;
  // streaming loads: the fp32 delta is read once
  f32x4 v0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(d));
  f32x4 v1 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(d + 4));
  for (int j0 = 0; j0 < p.top_k; j0 += FIN_KB) {
    const Route rt = load_route(p, t, j0);
    add_rows(rt, load_rows(p, rt, col), v0, v1);
  }
  store_out8(p, t, col, v0, v1);
}

// accumulator rows of EXP_CW floats; 16-byte chunk c of row tl sits at c ^ (tl & 31)
__device__ __forceinline__ int acc_chunk(int tl, int c) {
  return tl * (EXP_CW / 4) + (c ^ (tl & 31));
}

template <int NB>
struct Ring {  // operands of one 16-slot block, loaded D blocks ahead
  u32x4 fu[NB];  // u fragment: hi and lo of 4 ranks
  u32x2 fb[EXP_NCG][NB];  // B_le: the same 4 ranks of each of the wavefront's column groups
  uint32_t tw;   // the 4 token-row bytes around this lane's slot
  float f;       // fp16 carrier: 2^-k of this lane's slot
};

__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// The block loop of one wavefront.  PART: 16 * NB > rank, so some rank
// chunks are partly or wholly past the rank (those ranks are masked to zero in
// B, which may hold anything there; u is zero there).
// DUP: a block may hold a token twice, so accumulate with LDS atomics.
// F16: fp16 operands; each slot's products are multiplied by its 2^-k factor
// (fused into the accumulation as one FMA).
template <int NB, bool PART, bool DUP, bool F16>
__device__ __forceinline__ void expand_blocks(float* s_acc, const uint16_t* const* s_bp,
                                              const char* u2t, const char* tlt, const char* ft,
                                              int nblk, int R, int H, int h0) {
  constexpr int D = NB == 1 ? 4 : (NB == 2 ? 4 : (NB == 4 ? 2 : 1));  // ring depth
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kq = lane >> 4;
  // byte offsets of this lane inside a block's u record, B_le, token-row table
  const uint32_t uoff = lane * 16;
  uint32_t boff[EXP_NCG][NB];
  bool rin[NB];
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const int r4 = c * 16 + kq * 4;  // rank % 8 == 0: ranks r4 .. r4+3 are all in or all out
    rin[c] = r4 < R;
#pragma unroll
    for (int g = 0; g < EXP_NCG; ++g)
      // B_le is [hidden, rank]; column h0 + 16*(EXP_NCG*wave + g) + col, ranks r4 .. r4+3
      // (clamped into the column when past the rank; masked below)
      boff[g][c] = 2u * (static_cast<uint32_t>(h0 + 16 * (EXP_NCG * wave + g) + col) * R +
                         (rin[c] ? r4 : R - 4));
  }
  const uint32_t toff = (col >> 2) * 4;
  const int tsh = (col & 3) * 8;
  const int ca = 4 * EXP_NCG * wave + kq;  // accumulator chunk of group 0 (group g: + 4g)
  f32x4* acc4 = reinterpret_cast<f32x4*>(s_acc);

  // every block index is clamped to the last block, so each ring step issues
  // the same loads and the counter-based waits stay exact.  Buffer loads: the
  // per-lane offsets are constants, the block offset is a scalar.
  const __amdgpu_buffer_rsrc_t ursrc = buf_rsrc(u2t, static_cast<uint32_t>(nblk) * NB * 1024);
  const __amdgpu_buffer_rsrc_t trsrc = buf_rsrc(tlt, static_cast<uint32_t>(nblk) * 16);
  const __amdgpu_buffer_rsrc_t frsrc = buf_rsrc(ft, F16 ? static_cast<uint32_t>(nblk) * 64 : 0);
  const uint32_t bbytes = static_cast<uint32_t>(H) * R * 2;  // one B_le
  auto bptr = [&](int i) { return s_bp[min(i, nblk - 1)]; };
  auto load = [&](Ring<NB>& r, int i, const uint16_t* bsrc) {
    const uint32_t ic = static_cast<uint32_t>(min(i, nblk - 1));
#pragma unroll
    for (int c = 0; c < NB; ++c) r.fu[c] = buf_ld128(ursrc, c * 1024 + uoff, ic * NB * 1024);
    const __amdgpu_buffer_rsrc_t brsrc = buf_rsrc(uniform_ptr(bsrc), bbytes);
#pragma unroll
    for (int g = 0; g < EXP_NCG; ++g)
#pragma unroll
      for (int c = 0; c < NB; ++c) r.fb[g][c] = buf_ld64(brsrc, boff[g][c], 0);  // 512 B rows
    r.tw = buf_ld32(trsrc, toff, ic * 16);
    r.f = F16 ? __builtin_bit_cast(float, buf_ld32(frsrc, col * 4, ic * 64)) : 1.f;
  };
  auto mma = [&](const Ring<NB>& r, f32x4 (&acc)[EXP_NCG]) {
#pragma unroll
    for (int g = 0; g < EXP_NCG; ++g) {
      acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        u32x2 b4 = r.fb[g][c];
        if (PART && !rin[c]) b4 = u32x2{0, 0};
        const u32x4 fb = u32x4{b4.x, b4.y, b4.x, b4.y};
        // K = 32 runs over (4 ranks, hi|lo) of every lane group q: [B | B]
        // (16 columns x 32) times [u_hi ; u_lo] (32 x 16 slots)
        if constexpr (F16)
          acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, fb),
                                                          __builtin_bit_cast(f16x8, r.fu[c]),
                                                          acc[g], 0, 0, 0);
        else
          acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fb),
                                                           __builtin_bit_cast(bf16x8, r.fu[c]),
                                                           acc[g], 0, 0, 0);
      }
    }
  };
  // token row of this lane's slot; an empty slot or a block past the end goes
  // to spare row EXP_TT + col (written, never read back)
  auto row_of = [&](const Ring<NB>& r, bool valid) {
    const uint32_t tl = (r.tw >> tsh) & 0xFFu;
    return (valid && tl != 0xFFu) ? static_cast<int>(tl) : EXP_TT + col;
  };

  // Software pipeline, one block per step: the accumulator rows of block i
  // are read, block i+1 goes through the MFMAs and its ring slot is refilled
  // with block i+1+D, then block i is added and written back.  (Blocks i and
  // i+1 may share a token, so block i+1's rows are read only after block i's
  // writes.)  The B_le addresses of a round of D refills are read from LDS
  // together at its start.
  Ring<NB> ring[D];
#pragma unroll
  for (int d = 0; d < D; ++d) load(ring[d], d, bptr(d));
  f32x4 acc[EXP_NCG];
  mma(ring[0], acc);
  int tl = row_of(ring[0], true);  // nblk > 0
  float fs = ring[0].f;            // F16 only
  load(ring[0], D, bptr(D));
  for (int i0 = 0; i0 < nblk; i0 += D) {
    // the refill addresses of this pass over the ring, made scalar once (not inside the steps,
    // where each conversion would wait for the accumulator reads in flight)
    const uint16_t* bpr[D];
#pragma unroll
    for (int d = 0; d < D; ++d)
      bpr[d] = reinterpret_cast<const uint16_t*>(uniform_ptr(bptr(i0 + d + 1 + D)));
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int i = i0 + d;
      f32x4* a[EXP_NCG];
      f32x4 v[EXP_NCG];
#pragma unroll
      for (int g = 0; g < EXP_NCG; ++g) a[g] = acc4 + acc_chunk(tl, ca + 4 * g);
      if (!DUP) {
#pragma unroll
        for (int g = 0; g < EXP_NCG; ++g) v[g] = *a[g];
      }
      // the reads go first, so their latency runs under the next MFMAs and loads
      __builtin_amdgcn_sched_barrier(0);
      Ring<NB>& rn = ring[(d + 1) % D];  // holds block i+1
      f32x4 accn[EXP_NCG];
      mma(rn, accn);
      const int tln = row_of(rn, i + 1 < nblk);
      const float fsn = rn.f;
      load(rn, i + 1 + D, bpr[d]);
#pragma unroll
      for (int g = 0; g < EXP_NCG; ++g) {
        if (!DUP) {
          if (F16)
            *a[g] = v[g] + acc[g] * fs;  // one FMA per element; the product is exact
          else
            *a[g] = v[g] + acc[g];
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            atomicAdd(reinterpret_cast<float*>(a[g]) + q, F16 ? acc[g][q] * fs : acc[g][q]);
        }
      }
#pragma unroll
      for (int g = 0; g < EXP_NCG; ++g) acc[g] = accn[g];
      tl = tln;
      fs = fsn;
      // ring steps stay in order: left free, the scheduler hoists the MFMAs of
      // the whole round to its top, which then waits for every load in flight
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// 2 workgroups per CU (LDS) = 2 wavefronts per SIMD
template <int NB, bool PART, bool F16>
__global__ __launch_bounds__(NT_EXP, 2) void expand_kernel(ExpandArgs p) {
  __shared__ __attribute__((aligned(16))) float s_acc[(EXP_TT + 16) * EXP_CW];  // + spare rows
  __shared__ const uint16_t* s_bp[MAX_BLOCKS];  // B_le of each block
  __shared__ int s_tok[EXP_TT];                 // the tile's token ids

  // Workgroup order: the (column chunk, tile) pairs are taken in runs of
  // TB tiles -- all chunks of a run, tiles fastest -- and every XCD gets a
  // contiguous range of that order (the dispatcher deals workgroup ids to
  // the 8 XCDs in turn).  The u records of a run's tiles then stay in one
  // L2 while its chunks go by, and the run's tiles (mostly one adapter)
  // read each chunk of B_l together.
  constexpr int TB = 8;
  const int per = gridDim.x >> 3;
  const int lin = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  const int run = lin / (TB * p.nch), rem = lin % (TB * p.nch);
  const int ch = rem / TB, ti = run * TB + rem % TB;
  if (ti >= p.max_tiles) return;
  // the tile, its block count and its blocks' B_le addresses are read
  // together (all lie inside the workspace whatever the tile count); the
  // count decides afterwards whether the tile exists
  const int ntile = gld<int>(p.counters);
  const Tile tile = load_tile(p.tiles + ti);
  const int nblk0 = gld<int>(p.tinfo + 2 * ti);
  const int dup0 = gld<int>(p.tinfo + 2 * ti + 1);
  const int tid = threadIdx.x;
  const int64_t* bb = p.blk_b + static_cast<long>(ti) * p.maxblk;
  int64_t bpre[(MAX_BLOCKS + NT_EXP - 1) / NT_EXP];
#pragma unroll
  for (int k = 0; k < (MAX_BLOCKS + NT_EXP - 1) / NT_EXP; ++k) {
    const int i = tid + k * NT_EXP;
    if (i < p.maxblk) bpre[k] = gld<int64_t>(bb + i);
  }
  if (ti >= ntile) return;
  const int h0 = ch * EXP_CW;
  // the tile's token ids, for the write-out
  for (int i = tid; i < tile.count; i += NT_EXP) s_tok[i] = gld<int>(p.tok_list + tile.start + i);

  if (tile.bucket >= p.L) {  // no adapter: a +0 delta (plus the combine when finalizing)
    __syncthreads();  // s_tok
    write_tile(p, tile, h0, [](int, f32x4& v0, f32x4& v1) {
      v0 = f32x4{0.f, 0.f, 0.f, 0.f};
      v1 = f32x4{0.f, 0.f, 0.f, 0.f};
    }, s_tok);
    return;
  }
  const int nblk = nblk0;
  const bool dup = dup0 != 0;
#pragma unroll
  for (int k = 0; k < (MAX_BLOCKS + NT_EXP - 1) / NT_EXP; ++k) {
    const int i = tid + k * NT_EXP;
    if (i < nblk) s_bp[i] = reinterpret_cast<const uint16_t*>(bpre[k]);
  }
  for (int i = tid * 4; i < tile.count * EXP_CW; i += NT_EXP * 4)
    *reinterpret_cast<f32x4*>(s_acc + i) = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  if (nblk > 0) {
    const char* u2t = reinterpret_cast<const char*>(p.u2 + static_cast<long>(ti) * p.cap * NB * 32);
    const char* tlt = reinterpret_cast<const char*>(p.blk_tl + static_cast<long>(ti) * p.maxblk * 4);
    const char* ft = reinterpret_cast<const char*>(p.blk_f + static_cast<long>(ti) * p.maxblk * 16);
    if (dup)
      expand_blocks<NB, PART, true, F16>(s_acc, s_bp, u2t, tlt, ft, nblk, p.rank, p.H, h0);
    else
      expand_blocks<NB, PART, false, F16>(s_acc, s_bp, u2t, tlt, ft, nblk, p.rank, p.H, h0);
  }
  __syncthreads();
  const f32x4* a = reinterpret_cast<const f32x4*>(s_acc);
  write_tile(p, tile, h0, [&](int i, f32x4& v0, f32x4& v1) {
    const int tl = i / (EXP_CW / 8), c = (i % (EXP_CW / 8)) * 8;
    v0 = a[acc_chunk(tl, c / 4)];
    v1 = a[acc_chunk(tl, c / 4 + 1)];
  }, s_tok);
}

// ---------------------------------------------------------------------------
// FC1 LoRA delta: the same plan, list and shrink (unit routing weights), then
// an expand without accumulation -- every active slot owns its output row
//   out[perm[t*top_k+j]] = B_le @ u(t, j)        (u = scale * A_le @ act[row])
// ---------------------------------------------------------------------------
struct Fc1Args {
  const int32_t* btile;
  const int32_t* tex;
  const uint16_t* u2;
  const int64_t* w_ptr_b;
  long stride_b;
  const uint32_t* blk_tl;
  const int32_t* blk_row;
  const float* blk_f;
  void* out;
  long cap;
  int E, L, R, OF, maxblk, nch, out_kind;  // OF: output width (B_le rows)
};

// 8 consecutive output columns of one row, rounded once (streaming stores:
// the rows are written once and not read here)
__device__ __forceinline__ void store_out8c(void* out, int kind, long off, f32x4 v0, f32x4 v1) {
  if (kind == 1) {
    __builtin_nontemporal_store(v0, reinterpret_cast<f32x4*>(static_cast<float*>(out) + off));
    __builtin_nontemporal_store(v1, reinterpret_cast<f32x4*>(static_cast<float*>(out) + off + 4));
  } else if (kind == 2) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const h8 h = {static_cast<_Float16>(v0.x), static_cast<_Float16>(v0.y),
                  static_cast<_Float16>(v0.z), static_cast<_Float16>(v0.w),
                  static_cast<_Float16>(v1.x), static_cast<_Float16>(v1.y),
                  static_cast<_Float16>(v1.z), static_cast<_Float16>(v1.w)};
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, h),
                                reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + off));
  } else {
    const u32x4 w = {pack_bf16x2(v0.x, v0.y), pack_bf16x2(v0.z, v0.w), pack_bf16x2(v1.x, v1.y),
                     pack_bf16x2(v1.z, v1.w)};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + off));
  }
}

constexpr int FC1_MAX_BLK = 256;  // blocks of one (adapter, expert) listed in LDS at once

// One workgroup per (adapter l, expert e, chunk of CW output columns).
// Wavefront 0 lists the blocks of (l, e) in the tiles of adapter l (tile,
// block) into LDS; the four wavefronts then take them in turn.  Each
// wavefront holds that chunk of B_le in registers (per lane: 4 ranks of one
// column per 16-column group and rank chunk, the [B | B] operand of the FC2
// expand); per block it runs one v_mfma_f32_16x16x32 per group and rank chunk
// on [B | B] and the block's [u_hi ; u_lo] record.  The groups go in pairs
// whose MFMA rows are permuted so that lane (slot, q) receives 8 consecutive
// output columns of its slot's row from the pair and stores them as one
// 16-byte piece (pair p covers columns 32p .. 32p+31 of the chunk: MFMA row i
// of its first group is column 8(i/4) + i%4, of its second 8(i/4) + 4 + i%4).
// B_le is read from memory once per chunk.
template <int NB, bool PART, bool F16, int CW>
__global__ __launch_bounds__(256) void fc1_expand_kernel(Fc1Args p) {
  constexpr int NG = CW / 16;  // 16-column groups of the chunk (an even number)
  __shared__ int s_blk[FC1_MAX_BLK];  // (tile << 12) | block of each listed block
  __shared__ int s_nblk;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nch = p.OF / CW;
  const int ch = blockIdx.x % nch, le = blockIdx.x / nch;
  const int l = le / p.E, e = le % p.E;
  if (l >= p.L) return;
  const int t0 = gld<int>(p.btile + l), t1 = gld<int>(p.btile + l + 1);
  const int E1 = p.E + 1;
  const int col = lane & 15, kq = lane >> 4;
  const int h0 = ch * CW;

  // this lane's B_le fragments: group g, MFMA row col -> output column
  // h0 + 32 (g/2) + 8 (col/4) + 4 (g%2) + col%4, ranks 16 c + 4 kq .. + 3
  const char* ble = reinterpret_cast<const char*>(gld<int64_t>(p.w_ptr_b + e) + 2 * p.stride_b * l);
  const __amdgpu_buffer_rsrc_t brsrc =
      buf_rsrc(uniform_ptr(ble), static_cast<uint32_t>(p.OF) * p.R * 2);
  u32x2 fb[NG][NB];
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const int r4 = c * 16 + kq * 4;  // rank % 8 == 0: ranks r4 .. r4+3 all in or all out
    const bool rin = r4 < p.R;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int ocol = h0 + 32 * (g >> 1) + 8 * (col >> 2) + 4 * (g & 1) + (col & 3);
      const uint32_t off = 2u * (static_cast<uint32_t>(ocol) * p.R + (rin ? r4 : p.R - 4));
      fb[g][c] = buf_ld64(brsrc, off, 0);
      if (PART && !rin) fb[g][c] = u32x2{0, 0};
    }
  }

  // the block list of (l, e): one lane per tile, a scan, then the entries
  if (wave == 0) {
    int n = 0;
    for (int tb = t0; tb < t1; tb += 64) {
      const int ti = tb + lane;
      int b0 = 0, cnt = 0;
      if (ti < t1) {
        b0 = gld<int>(p.tex + static_cast<long>(ti) * E1 + e);
        cnt = gld<int>(p.tex + static_cast<long>(ti) * E1 + e + 1) - b0;
      }
      int incl = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      for (int i = 0; i < cnt; ++i) {
        const int slot = n + incl - cnt + i;
        if (slot < FC1_MAX_BLK) s_blk[slot] = ((ti - t0) << 12) | (b0 + i);
      }
      n += __shfl(incl, 63, 64);
    }
    if (lane == 0) s_nblk = n;
  }
  __syncthreads();
  const int nblk = s_nblk;

  // one block's operands: its u record fragments and this lane's slot (row,
  // whether the slot is real, the fp16 factor)
  struct Blk {
    u32x4 fu[NB];
    uint32_t tlw;
    int row;
    float fs;
  };
  const int slot = col;
  auto fetch = [&](int ti, int bi) {
    Blk q;
    const long tb = static_cast<long>(ti) * p.maxblk + bi;
    const uint16_t* rec = p.u2 + (static_cast<long>(ti) * p.cap + bi * 16) * NB * 32;
#pragma unroll
    for (int c = 0; c < NB; ++c) q.fu[c] = gld<u32x4>(rec + c * 512 + lane * 8);
    q.tlw = gld<uint32_t>(p.blk_tl + tb * 4 + (slot >> 2));
    q.row = gld<int>(p.blk_row + tb * 16 + slot);
    q.fs = F16 ? gld<float>(p.blk_f + tb * 16 + slot) : 1.f;
    return q;
  };
  auto compute = [&](const Blk& q) {
    const bool real = ((q.tlw >> (8 * (slot & 3))) & 0xFFu) != 0xFFu;
    const long row = q.row;
#pragma unroll
    for (int gp = 0; gp < NG / 2; ++gp) {
      f32x4 acc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NB; ++c) {
          const u32x2 b2 = fb[2 * gp + h][c];
          const u32x4 a4 = u32x4{b2.x, b2.y, b2.x, b2.y};
          if constexpr (F16)
            acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a4),
                                                            __builtin_bit_cast(f16x8, q.fu[c]),
                                                            acc[h], 0, 0, 0);
          else
            acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a4),
                                                             __builtin_bit_cast(bf16x8, q.fu[c]),
                                                             acc[h], 0, 0, 0);
        }
        if (F16) acc[h] = acc[h] * q.fs;  // the slot's 2^-k: exact
      }
      // lane (slot, kq): columns 32 gp + 8 kq .. + 7 of its slot's row
      if (real) store_out8c(p.out, p.out_kind, row * p.OF + h0 + 32 * gp + 8 * kq, acc[0], acc[1]);
    }
  };
  if (nblk <= FC1_MAX_BLK) {
    // the next block's operands are loaded while this one is computed and
    // stored (the last step reloads the last block; not computed)
    if (wave < nblk) {
      Blk cur = fetch(t0 + (s_blk[wave] >> 12), s_blk[wave] & 4095);
      for (int j = wave; j < nblk; j += 4) {
        const int v = s_blk[min(j + 4, nblk - 1)];
        const Blk nxt = fetch(t0 + (v >> 12), v & 4095);
        compute(cur);
        cur = nxt;
      }
    }
  } else {  // more blocks than the list holds: walk the tiles directly
    int j = 0;
    for (int ti = t0; ti < t1; ++ti) {
      const int b0 = gld<int>(p.tex + static_cast<long>(ti) * E1 + e);
      const int b1 = gld<int>(p.tex + static_cast<long>(ti) * E1 + e + 1);
      for (int bi = b0; bi < b1; ++bi, ++j)
        if ((j & 3) == wave) compute(fetch(ti, bi));
    }
  }
}

// +0 rows of the FC1 delta: one wavefront per slot; a slot with a row in
// [0, padded_rows) whose token has no adapter (id outside [0, L)) or whose
// expert lies outside [0, E) gets a zero row (the expand writes the others)
__global__ __launch_bounds__(256) void fc1_zero_rows_kernel(const int32_t* perm,
                                                            const int32_t* topk_ids,
                                                            const int32_t* lora_ids, long nslot,
                                                            int top_k, int E, int L,
                                                            int padded_rows, void* out,
                                                            long row_bytes) {
  const long sl = (static_cast<long>(blockIdx.x) * 256 + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (sl >= nslot) return;
  const int r = gld<int>(perm + sl);
  if (r < 0 || r >= padded_rows) return;
  const int l = gld<int>(lora_ids + sl / top_k), e = gld<int>(topk_ids + sl);
  if (l >= 0 && l < L && e >= 0 && e < E) return;
  char* o = static_cast<char*>(out) + static_cast<long>(r) * row_bytes;
  for (long b = lane * 16; b < row_bytes; b += 64 * 16)
    __builtin_nontemporal_store(u32x4{0, 0, 0, 0}, reinterpret_cast<u32x4*>(o + b));
}

int num_cus() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    return 256;
  return v;
}

}  // namespace
}  // namespace mi

extern "C" size_t mi_moe_fc2_lora_delta_workspace_size(int64_t num_tokens, int64_t top_k,
                                                       int64_t num_experts, int64_t num_adapters,
                                                       int64_t rank) {
  if (num_tokens < 0 || top_k < 1 || top_k > mi::MAX_TOPK || num_experts < 1 ||
      num_adapters < 0 || rank < 1)
    return 0;
  return mi::layout(num_tokens, top_k, num_experts, num_adapters, rank).total;
}

namespace mi {
namespace {
size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }
}  // namespace
}  // namespace mi

extern "C" size_t mi_moe_fc2_finalize_workspace_size(int64_t num_tokens, int64_t top_k,
                                                     int64_t num_experts, int64_t num_adapters,
                                                     int64_t rank, int64_t hidden_size) {
  const size_t d = mi_moe_fc2_lora_delta_workspace_size(num_tokens, top_k, num_experts,
                                                        num_adapters, rank);
  if (d == 0 || hidden_size < 1) return 0;
  return mi::align256(d) + static_cast<size_t>(num_tokens) * static_cast<size_t>(hidden_size) * 4;
}

namespace mi {
namespace {

// What the plan, list and shrink launches leave for an expand: the workspace
// sections and the launch shape.
struct Front {
  Layout ly;
  uint8_t* ws;
  uint16_t* u2;
  int32_t *tok_list, *counters, *tinfo, *btile, *tex, *blk_row;
  Tile* tiles;
  int64_t* blk_b;
  uint32_t* blk_tl;
  float* blk_f;
  int ntiles, nb;
  bool f16;
};

// Validation shared by the FC2 and FC1 deltas (messages name `what`), then
// the plan, list and shrink launches.  `act` is [padded_rows, in_width] (I for
// FC2, hidden for FC1); B_le is [out_width, rank] (H for FC2, 2I for FC1);
// topk_weights may be NULL (unit weights).
mi_status check_front(const char* what, const void* act, int64_t padded_rows, int64_t in_width,
                      const int32_t* perm, const int64_t* w_ptr_a, int64_t lora_stride_a,
                      const int64_t* w_ptr_b, int64_t lora_stride_b, const int32_t* topk_ids,
                      const int32_t* lora_ids, int64_t T, int64_t top_k, int64_t E, int64_t L,
                      int64_t rank, int64_t out_width, mi_dtype lora_dtype, mi_dtype out_dtype,
                      void* out) {
  MI_REQUIRE(top_k >= 1 && top_k <= MAX_TOPK, "%s: top_k must be in [1, %d]", what, MAX_TOPK);
  MI_REQUIRE(T >= 0 && T * top_k < (1LL << 24), "%s: num_tokens * top_k must be < 2^24", what);
  MI_REQUIRE(E >= 1 && E <= MAX_EXPERTS, "%s: num_experts must be in [1, %d]", what,
             MAX_EXPERTS);
  MI_REQUIRE(L >= 0 && L <= MAX_ADAPTERS, "%s: num_adapters must be in [0, %d]", what,
             MAX_ADAPTERS);
  MI_REQUIRE(rank >= 8 && rank <= 128 && rank % 8 == 0,
             "%s: rank must be a multiple of 8 in [8, 128] (got %lld)", what, (long long)rank);
  MI_REQUIRE(in_width >= 8 && in_width % 8 == 0 && in_width < (1 << 30),
             "%s: the activation width must be a positive multiple of 8 (got %lld)", what,
             (long long)in_width);
  MI_REQUIRE(out_width >= 1 && out_width < (1 << 30), "%s: output width out of range", what);
  // one B_le block is addressed through a 32-bit buffer range
  MI_REQUIRE_SUPPORTED(out_width * rank * 2 < (1LL << 32),
                       "%s: one B block (%lld x %lld rank, 16-bit) must stay below 4 GiB", what,
                       (long long)out_width, (long long)rank);
  MI_REQUIRE_SUPPORTED(out_width % EXP_CW == 0, "%s: the output width must be a multiple of %d "
                       "(got %lld)", what, EXP_CW, (long long)out_width);
  MI_REQUIRE(lora_stride_a >= 0 && lora_stride_a % 8 == 0 && lora_stride_b >= 0 &&
                 lora_stride_b % 8 == 0,
             "%s: lora strides must be non-negative multiples of 8 elements (16-byte aligned "
             "adapter blocks)", what);
  MI_REQUIRE(padded_rows >= 0 && padded_rows < (1LL << 31), "%s: padded_rows out of range",
             what);
  MI_REQUIRE(lora_dtype == MI_BF16 || lora_dtype == MI_F16,
             "%s: lora_dtype must be bf16 or fp16", what);
  MI_REQUIRE(out_dtype == MI_BF16 || out_dtype == MI_F32 || out_dtype == MI_F16,
             "%s: out_dtype must be bf16, fp16 or fp32", what);
  if (T == 0) return MI_OK;
  MI_REQUIRE(out != nullptr, "%s: out is null", what);
  MI_REQUIRE(aligned16(out), "%s: out must be 16-byte aligned", what);
  MI_REQUIRE(lora_ids != nullptr && topk_ids != nullptr && perm != nullptr,
             "%s: index/weight tensors must be non-null", what);
  if (L > 0)
    MI_REQUIRE((act != nullptr || padded_rows == 0) && w_ptr_a != nullptr && w_ptr_b != nullptr,
               "%s: act and the pointer tables must be non-null", what);
  MI_REQUIRE(aligned16(act), "%s: activation rows must be 16-byte aligned", what);
  return MI_OK;
}

mi_status run_front(const char* what, const void* act, int64_t padded_rows, int64_t in_width,
                    const int32_t* perm, const int64_t* w_ptr_a, int64_t lora_stride_a,
                    const int64_t* w_ptr_b, int64_t lora_stride_b, const int32_t* topk_ids,
                    const float* topk_weights, const int32_t* lora_ids, int64_t T, int64_t top_k,
                    int64_t E, int64_t L, int64_t rank, int64_t out_width, mi_dtype lora_dtype,
                    float scale, mi_dtype out_dtype, void* out, void* workspace,
                    size_t workspace_bytes, hipStream_t s, Front& f) {
  mi_status st0 = check_front(what, act, padded_rows, in_width, perm, w_ptr_a, lora_stride_a,
                              w_ptr_b, lora_stride_b, topk_ids, lora_ids, T, top_k, E, L, rank,
                              out_width, lora_dtype, out_dtype, out);
  if (st0 != MI_OK || T == 0) return st0;
  f.ly = layout(T, top_k, E, L, rank);
  const Layout& ly = f.ly;
  MI_REQUIRE(workspace != nullptr && workspace_bytes >= ly.total,
             "%s: workspace needs %zu bytes (got %zu)", what, ly.total, workspace_bytes);
  MI_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255) == 0,
             "%s: workspace must be 256-byte aligned", what);

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  f.ws = ws;
  f.u2 = reinterpret_cast<uint16_t*>(ws + ly.u2);
  f.tok_list = reinterpret_cast<int32_t*>(ws + ly.tok_list);
  f.tiles = reinterpret_cast<Tile*>(ws + ly.tiles);
  f.counters = reinterpret_cast<int32_t*>(ws + ly.counters);
  int64_t* blk_a = reinterpret_cast<int64_t*>(ws + ly.blk_a);
  f.blk_b = reinterpret_cast<int64_t*>(ws + ly.blk_b);
  f.blk_row = reinterpret_cast<int32_t*>(ws + ly.blk_row);
  float* blk_w = reinterpret_cast<float*>(ws + ly.blk_w);
  f.blk_f = reinterpret_cast<float*>(ws + ly.blk_f);
  f.f16 = lora_dtype == MI_F16;
  f.blk_tl = reinterpret_cast<uint32_t*>(ws + ly.blk_tl);
  f.tinfo = reinterpret_cast<int32_t*>(ws + ly.tinfo);
  const int tt = tile_tokens(top_k);
  f.ntiles = static_cast<int>(max_tiles(T, top_k, L));
  f.btile = reinterpret_cast<int32_t*>(ws + ly.btile);
  f.tex = reinterpret_cast<int32_t*>(ws + ly.tex);
  f.nb = rank_chunks(rank);
  const int ntiles = f.ntiles, nb = f.nb;
  const bool f16 = f.f16;
  uint16_t* u2 = f.u2;
  float* blk_f = f.blk_f;

  PlanArgs pa{lora_ids, static_cast<int>(T), static_cast<int>(L), tt, f.tok_list, f.tiles,
              f.counters, f.btile};
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, s, pa);
  mi_status st = launch_status(what);
  if (st != MI_OK || L == 0) return st;

  const SlotSrc src{f.tok_list, perm, topk_ids, topk_weights, static_cast<int>(top_k),
                    static_cast<int>(padded_rows), static_cast<int>(E)};
  ListArgs la{src, f.tiles, f.counters, topk_weights, w_ptr_a, static_cast<long>(lora_stride_a),
              w_ptr_b, static_cast<long>(lora_stride_b), blk_a, f.blk_b, f.blk_tl, f.blk_row,
              blk_w, f.tinfo, f.tex, static_cast<int>(L), ly.maxblk, scale};
  hipLaunchKernelGGL(list_kernel, dim3(ntiles), dim3(NT_DELTA), 0, s, la);
  st = launch_status(what);
  if (st != MI_OK) return st;

  // A_le held in LDS when it fits: one workgroup per (adapter, expert, part);
  // up to 64 KB of A_le two workgroups per CU, up to 128 KB one
  const bool by_le = nb <= 2 && 16 * nb * in_width <= SLE_AMAX_BIG && in_width % 128 == 0;
  const bool big_a = 16 * nb * in_width > SLE_AMAX;
  if (by_le) {
    const long le = L * E;
    // parts: the tiles of an adapter split S ways when the pairs alone would not
    // fill every workgroup slot of the chip
    const int S = le >= (big_a ? 1L : 2L) * num_cus() ? 1 : 2;
    MI_REQUIRE(le * S < (1L << 31), "%s: problem too large", what);
    ShrinkLeArgs sa{static_cast<const uint16_t*>(act), w_ptr_a, static_cast<long>(lora_stride_a),
                    f.btile, f.tex, f.blk_row, blk_w, u2, blk_f, ly.cap,
                    static_cast<int>(in_width), static_cast<int>(E), static_cast<int>(L),
                    static_cast<int>(rank), ly.maxblk, S};
    const dim3 g(static_cast<unsigned>(le * S)), b(256);
    switch (nb * 4 + (f16 ? 2 : 0) + (big_a ? 1 : 0)) {
      case 4: hipLaunchKernelGGL((shrink_le_kernel<1, false, SLE_AMAX>), g, b, 0, s, sa); break;
      case 5: hipLaunchKernelGGL((shrink_le_kernel<1, false, SLE_AMAX_BIG>), g, b, 0, s, sa); break;
      case 6: hipLaunchKernelGGL((shrink_le_kernel<1, true, SLE_AMAX>), g, b, 0, s, sa); break;
      case 7: hipLaunchKernelGGL((shrink_le_kernel<1, true, SLE_AMAX_BIG>), g, b, 0, s, sa); break;
      case 8: hipLaunchKernelGGL((shrink_le_kernel<2, false, SLE_AMAX>), g, b, 0, s, sa); break;
      case 9: hipLaunchKernelGGL((shrink_le_kernel<2, false, SLE_AMAX_BIG>), g, b, 0, s, sa); break;
      case 10: hipLaunchKernelGGL((shrink_le_kernel<2, true, SLE_AMAX>), g, b, 0, s, sa); break;
      default: hipLaunchKernelGGL((shrink_le_kernel<2, true, SLE_AMAX_BIG>), g, b, 0, s, sa); break;
    }
  } else {
    const int bpt = (ly.maxblk + SHR_WAVES - 1) / SHR_WAVES;  // shrink workgroups per tile
    const long swg = static_cast<long>(ntiles) * bpt;
    MI_REQUIRE(swg < (1L << 31), "%s: problem too large", what);
    ShrinkArgs sa{static_cast<const uint16_t*>(act), f.tiles, f.counters, blk_a, f.blk_row, blk_w,
                  f.tinfo, u2, blk_f, ly.cap, static_cast<int>(in_width), static_cast<int>(L),
                  static_cast<int>(rank), ly.maxblk, bpt};
    const dim3 sgrid(static_cast<unsigned>(swg)), sblock(64 * SHR_WAVES);
    switch (nb * 2 + (f16 ? 1 : 0)) {
      case 2: hipLaunchKernelGGL((shrink_kernel<1, false>), sgrid, sblock, 0, s, sa); break;
      case 3: hipLaunchKernelGGL((shrink_kernel<1, true>), sgrid, sblock, 0, s, sa); break;
      case 4: hipLaunchKernelGGL((shrink_kernel<2, false>), sgrid, sblock, 0, s, sa); break;
      case 5: hipLaunchKernelGGL((shrink_kernel<2, true>), sgrid, sblock, 0, s, sa); break;
      case 8: hipLaunchKernelGGL((shrink_kernel<4, false>), sgrid, sblock, 0, s, sa); break;
      case 9: hipLaunchKernelGGL((shrink_kernel<4, true>), sgrid, sblock, 0, s, sa); break;
      case 16: hipLaunchKernelGGL((shrink_kernel<8, false>), sgrid, sblock, 0, s, sa); break;
      default: hipLaunchKernelGGL((shrink_kernel<8, true>), sgrid, sblock, 0, s, sa); break;
    }
  }
  return launch_status(what);
}

// The delta and, when fc2 is given, the finalize: both entry points below.
mi_status run_delta(const char* what, const void* act, int64_t padded_rows, int64_t inter_size,
                    const int32_t* perm, const int64_t* w_ptr_a, int64_t lora_stride_a,
                    const int64_t* w_ptr_b, int64_t lora_stride_b, const int32_t* topk_ids,
                    const float* topk_weights, const int32_t* lora_ids, int64_t T, int64_t top_k,
                    int64_t E, int64_t L, int64_t rank, int64_t H, mi_dtype lora_dtype,
                    float scale, const void* fc2, mi_dtype fc2_dtype, mi_dtype out_dtype,
                    void* out, void* workspace, size_t workspace_bytes, void* stream) {
  MI_REQUIRE(topk_weights != nullptr || T == 0, "%s: topk_weights is null", what);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // with no activation rows every slot is inactive: the delta is +0 and the
  // finalize has no FC2 row to combine, so neither act nor fc2 is read
  if (padded_rows == 0) fc2 = nullptr;
  Front f;
  mi_status st = run_front(what, act, padded_rows, inter_size, perm, w_ptr_a, lora_stride_a,
                           w_ptr_b, lora_stride_b, topk_ids, topk_weights, lora_ids, T, top_k, E,
                           L, rank, H, lora_dtype, scale, out_dtype, out, workspace,
                           workspace_bytes, s, f);
  if (st != MI_OK || T == 0) return st;
  const Layout& ly = f.ly;
  uint8_t* ws = f.ws;
  const int ntiles = f.ntiles, nb = f.nb;
  const bool f16 = f.f16;
  uint16_t* u2 = f.u2;
  int32_t* tok_list = f.tok_list;
  Tile* tiles = f.tiles;
  int32_t* counters = f.counters;
  int64_t* blk_b = f.blk_b;
  uint32_t* blk_tl = f.blk_tl;
  float* blk_f = f.blk_f;
  int32_t* tinfo = f.tinfo;

  const int nch = static_cast<int>(H / EXP_CW);
  // Finalize in two passes when the workspace also holds an fp32 [T, H] delta:
  // the expand writes the delta there and finalize_combine_kernel reads whole
  // FC2 rows.  Otherwise the expand's write-out adds the rows itself.
  const size_t scratch_off = align256(ly.total);
  const bool two_pass = fc2 != nullptr &&
                        workspace_bytes >= scratch_off + static_cast<size_t>(T) * H * 4 &&
                        T * (H / 8) < (1LL << 38);  // combine grid below 2^30 workgroups
  float* scratch = two_pass ? reinterpret_cast<float*>(ws + scratch_off) : nullptr;
  const int out_kind = out_dtype == MI_F32 ? 1 : (out_dtype == MI_F16 ? 2 : 0);
  ExpandArgs ea{tok_list, tiles, counters, u2, blk_b, blk_tl, blk_f, tinfo,
                two_pass ? static_cast<void*>(scratch) : out, ly.cap,
                static_cast<int>(L), static_cast<int>(H), static_cast<int>(rank), ly.maxblk,
                ntiles, nch, two_pass ? 1 : out_kind,
                two_pass ? nullptr : fc2, perm, topk_weights,
                fc2_dtype == MI_F32 ? 1 : (fc2_dtype == MI_F16 ? 2 : 0),
                static_cast<int>(top_k), static_cast<int>(padded_rows)};
  // whole runs of 8 tiles x nch chunks, rounded to a multiple of the 8 XCDs
  const long ewg = ((static_cast<long>(ntiles) + 7) / 8 * 8 * nch + 7) & ~7L;
  MI_REQUIRE(ewg < (1L << 31), "bgmv_moe_gemm2_lora_delta: problem too large");
  const dim3 egrid(static_cast<unsigned>(ewg)), eblock(NT_EXP);
  const bool part = rank != 16 * nb;  // rank chunks past the rank are masked
  switch (nb * 4 + (part ? 2 : 0) + (f16 ? 1 : 0)) {
#define MI_EXPAND_CASE(NB_, PART_, F16_)                                                 \
  case NB_ * 4 + (PART_ ? 2 : 0) + (F16_ ? 1 : 0):                                        \
    hipLaunchKernelGGL((expand_kernel<NB_, PART_, F16_>), egrid, eblock, 0, s, ea); break;
    MI_EXPAND_CASE(1, false, false) MI_EXPAND_CASE(1, false, true)
    MI_EXPAND_CASE(1, true, false) MI_EXPAND_CASE(1, true, true)
    MI_EXPAND_CASE(2, false, false) MI_EXPAND_CASE(2, false, true)
    MI_EXPAND_CASE(2, true, false) MI_EXPAND_CASE(2, true, true)
    MI_EXPAND_CASE(4, false, false) MI_EXPAND_CASE(4, false, true)
    MI_EXPAND_CASE(4, true, false) MI_EXPAND_CASE(4, true, true)
    MI_EXPAND_CASE(8, false, false) MI_EXPAND_CASE(8, false, true)
    MI_EXPAND_CASE(8, true, false) MI_EXPAND_CASE(8, true, true)
#undef MI_EXPAND_CASE
    default: MI_REQUIRE(false, "bgmv_moe_gemm2_lora_delta: no expand variant (rank %lld)",
                        (long long)rank);
  }
  st = launch_status("bgmv_moe_gemm2_lora_delta (expand)");
  if (st != MI_OK || !two_pass) return st;
  ExpandArgs fa = ea;
  fa.out = out;
  fa.out_kind = out_kind;
  fa.fc2 = fc2;
  const long items = T * (H / 8);
  hipLaunchKernelGGL(finalize_combine_kernel, dim3(static_cast<unsigned>((items + 255) / 256)),
                     dim3(256), 0, s, fa, static_cast<const float*>(scratch), static_cast<int>(T));
  return launch_status("moe_fc2_finalize_lora (combine)");
}


// FC1 LoRA delta: the shared front end, then the expand by (adapter, expert)
// and the +0 rows of the slots without adapter or with an invalid expert.
mi_status run_fc1(const void* act, int64_t padded_rows, int64_t hidden, const int32_t* perm,
                  const int64_t* w_ptr_a, int64_t lora_stride_a, const int64_t* w_ptr_b,
                  int64_t lora_stride_b, const int32_t* topk_ids, const int32_t* lora_ids,
                  int64_t T, int64_t top_k, int64_t E, int64_t L, int64_t rank, int64_t OF,
                  mi_dtype lora_dtype, float scale, mi_dtype out_dtype, void* out,
                  void* workspace, size_t workspace_bytes, void* stream) {
  const char* what = "moe_fc1_lora_delta";
  hipStream_t s = static_cast<hipStream_t>(stream);
  Front f;
  mi_status st = run_front(what, act, padded_rows, hidden, perm, w_ptr_a, lora_stride_a, w_ptr_b,
                           lora_stride_b, topk_ids, nullptr, lora_ids, T, top_k, E, L, rank, OF,
                           lora_dtype, scale, out_dtype, out, workspace, workspace_bytes, s, f);
  if (st != MI_OK || T == 0 || padded_rows == 0) return st;
  const int out_kind = out_dtype == MI_F32 ? 1 : (out_dtype == MI_F16 ? 2 : 0);
  const long esize = out_dtype == MI_F32 ? 4 : 2;
  if (L > 0) {
    // chunk width: 64 VGPRs of B fragments per lane (512 columns at rank <= 16)
    const int cw = f.nb == 1 ? 512 : f.nb == 2 ? 256 : f.nb == 4 ? 128 : 64;
    const int cwu = static_cast<int>(OF % cw == 0 ? cw : EXP_CW);  // OF % 128 == 0
    const long wg = L * E * (OF / cwu);
    MI_REQUIRE(wg < (1L << 31), "%s: problem too large", what);
    Fc1Args fa{f.btile, f.tex, f.u2, w_ptr_b, static_cast<long>(lora_stride_b), f.blk_tl,
               f.blk_row, f.blk_f, out, f.ly.cap, static_cast<int>(E), static_cast<int>(L),
               static_cast<int>(rank), static_cast<int>(OF), f.ly.maxblk,
               static_cast<int>(OF / cwu), out_kind};
    const bool part = rank != 16 * f.nb;
    const dim3 g(static_cast<unsigned>(wg)), b(256);
    const bool full = cwu == cw;
    switch (f.nb * 4 + (part ? 2 : 0) + (f.f16 ? 1 : 0)) {
#define MI_FC1_CASE(NB_, PART_, F16_)                                                        \
  case NB_ * 4 + (PART_ ? 2 : 0) + (F16_ ? 1 : 0):                                            \
    if (full)                                                                                 \
      hipLaunchKernelGGL((fc1_expand_kernel<NB_, PART_, F16_,                                 \
                                            NB_ == 1 ? 512 : NB_ == 2 ? 256 : NB_ == 4 ? 128 : 64>), \
                         g, b, 0, s, fa);                                                     \
    else                                                                                      \
      hipLaunchKernelGGL((fc1_expand_kernel<NB_, PART_, F16_, (NB_ == 8 ? 64 : 128)>), g, b, 0, \
                         s, fa);                                                              \
    break;
      MI_FC1_CASE(1, false, false) MI_FC1_CASE(1, false, true)
      MI_FC1_CASE(1, true, false) MI_FC1_CASE(1, true, true)
      MI_FC1_CASE(2, false, false) MI_FC1_CASE(2, false, true)
      MI_FC1_CASE(2, true, false) MI_FC1_CASE(2, true, true)
      MI_FC1_CASE(4, false, false) MI_FC1_CASE(4, false, true)
      MI_FC1_CASE(4, true, false) MI_FC1_CASE(4, true, true)
      MI_FC1_CASE(8, false, false) MI_FC1_CASE(8, false, true)
      MI_FC1_CASE(8, true, false) MI_FC1_CASE(8, true, true)
#undef MI_FC1_CASE
      default: MI_REQUIRE(false, "%s: no expand variant (rank %lld)", what, (long long)rank);
    }
    st = launch_status(what);
    if (st != MI_OK) return st;
  }
  const long nslot = T * top_k;
  hipLaunchKernelGGL(fc1_zero_rows_kernel, dim3(static_cast<unsigned>((nslot + 3) / 4)), dim3(256),
                     0, s, perm, topk_ids, lora_ids, nslot, static_cast<int>(top_k),
                     static_cast<int>(E), static_cast<int>(L), static_cast<int>(padded_rows), out,
                     OF * esize);
  return launch_status(what);
}
}  // namespace
}  // namespace mi

extern "C" mi_status mi_moe_fc2_lora_delta(
    const void* act, int64_t padded_rows, int64_t inter_size, const int32_t* perm,
    const int64_t* w_ptr_a, int64_t lora_stride_a, const int64_t* w_ptr_b, int64_t lora_stride_b,
    const int32_t* topk_ids, const float* topk_weights, const int32_t* lora_ids, int64_t T,
    int64_t top_k, int64_t E, int64_t L, int64_t rank, int64_t H, mi_dtype lora_dtype, float scale,
    mi_dtype out_dtype, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  mi::clear_error();
  return mi::run_delta("bgmv_moe_gemm2_lora_delta", act, padded_rows, inter_size, perm, w_ptr_a,
                       lora_stride_a, w_ptr_b, lora_stride_b, topk_ids, topk_weights, lora_ids, T,
                       top_k, E, L, rank, H, lora_dtype, scale, nullptr, MI_BF16, out_dtype, out,
                       workspace, workspace_bytes, stream);
}

extern "C" mi_status mi_moe_fc2_finalize_lora(
    const void* fc2, mi_dtype fc2_dtype, const void* act, int64_t padded_rows,
    int64_t inter_size, const int32_t* perm, const int64_t* w_ptr_a, int64_t lora_stride_a,
    const int64_t* w_ptr_b, int64_t lora_stride_b, const int32_t* topk_ids,
    const float* topk_weights, const int32_t* lora_ids, int64_t T, int64_t top_k, int64_t E,
    int64_t L, int64_t rank, int64_t H, mi_dtype lora_dtype, float scale, mi_dtype out_dtype,
    void* out, void* workspace, size_t workspace_bytes, void* stream) {
  mi::clear_error();
  MI_REQUIRE(fc2_dtype == MI_BF16 || fc2_dtype == MI_F16 || fc2_dtype == MI_F32,
             "moe_fc2_finalize_lora: fc2_out dtype must be bf16, fp16 or fp32");
  if (T > 0 && padded_rows > 0) {
    MI_REQUIRE(fc2 != nullptr, "moe_fc2_finalize_lora: fc2_out is null");
    MI_REQUIRE(mi::aligned16(fc2), "moe_fc2_finalize_lora: fc2_out must be 16-byte aligned");
  }
  return mi::run_delta("moe_fc2_finalize_lora", act, padded_rows, inter_size, perm, w_ptr_a,
                       lora_stride_a, w_ptr_b, lora_stride_b, topk_ids, topk_weights, lora_ids, T,
                       top_k, E, L, rank, H, lora_dtype, scale, fc2, fc2_dtype, out_dtype, out,
                       workspace, workspace_bytes, stream);
}

extern "C" size_t mi_moe_fc1_lora_delta_workspace_size(int64_t num_tokens, int64_t top_k,
                                                       int64_t num_experts, int64_t num_adapters,
                                                       int64_t rank) {
  return mi_moe_fc2_lora_delta_workspace_size(num_tokens, top_k, num_experts, num_adapters, rank);
}

extern "C" mi_status mi_moe_fc1_lora_delta(
    const void* act, int64_t padded_rows, int64_t hidden_size, const int32_t* perm,
    const int64_t* w_ptr_a, int64_t lora_stride_a, const int64_t* w_ptr_b, int64_t lora_stride_b,
    const int32_t* topk_ids, const int32_t* lora_ids, int64_t T, int64_t top_k, int64_t E,
    int64_t L, int64_t rank, int64_t out_features, mi_dtype lora_dtype, float scale,
    mi_dtype out_dtype, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  mi::clear_error();
  return mi::run_fc1(act, padded_rows, hidden_size, perm, w_ptr_a, lora_stride_a, w_ptr_b,
                     lora_stride_b, topk_ids, lora_ids, T, top_k, E, L, rank, out_features,
                     lora_dtype, scale, out_dtype, out, workspace, workspace_bytes, stream);
}

namespace mi {
namespace {

constexpr int SCRATCH_MAX_DEVICES = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[SCRATCH_MAX_DEVICES];  // device address of `scratch`, per device

// The current device's address of `scratch`, looked up once per device
// (hipGetSymbolAddress: no allocation).
mi_status scratch_address(const char* what, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES) {
    set_error("%s: no usable current device (%s)", what, hipGetErrorString(e));
    return MI_EHIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      set_error("%s: hipGetSymbolAddress of the scratch array failed (%s)", what,
                hipGetErrorString(e));
      return MI_EHIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MI_OK;
}

}  // namespace
}  // namespace mi

extern "C" mi_status mi_moe_fc2_lora_delta_noalloc(
    const void* act, int64_t padded_rows, int64_t inter_size, const int32_t* perm,
    const int64_t* w_ptr_a, int64_t lora_stride_a, const int64_t* w_ptr_b, int64_t lora_stride_b,
    const int32_t* topk_ids, const float* topk_weights, const int32_t* lora_ids, int64_t T,
    int64_t top_k, int64_t E, int64_t L, int64_t rank, int64_t H, mi_dtype lora_dtype, float scale,
    mi_dtype out_dtype, void* out, void* stream) {
  using namespace mi;
  const char* what = "moe_fc2_lora_delta_noalloc";
  clear_error();
  mi_status st = check_front(what, act, padded_rows, inter_size, perm, w_ptr_a, lora_stride_a,
                             w_ptr_b, lora_stride_b, topk_ids, lora_ids, T, top_k, E, L, rank, H,
                             lora_dtype, out_dtype, out);
  if (st != MI_OK || T == 0) return st;
  MI_REQUIRE(topk_weights != nullptr, "%s: topk_weights is null", what);
  const size_t need = layout(T, top_k, E, L, rank).total;
  MI_REQUIRE_SUPPORTED(need <= MI_DELTA_SCRATCH_BYTES,
                       "%s: this problem needs %zu bytes of scratch; the fixed array holds %zu "
                       "(use mi_moe_fc2_lora_delta with a workspace)", what, need,
                       static_cast<size_t>(MI_DELTA_SCRATCH_BYTES));
  void* ws = nullptr;
  st = scratch_address(what, &ws);
  if (st != MI_OK) return st;
  // the delta writes every workspace entry it reads, so nothing needs clearing
  return run_delta(what, act, padded_rows, inter_size, perm, w_ptr_a, lora_stride_a, w_ptr_b,
                   lora_stride_b, topk_ids, topk_weights, lora_ids, T, top_k, E, L, rank, H,
                   lora_dtype, scale, nullptr, MI_BF16, out_dtype, out, ws,
                   MI_DELTA_SCRATCH_BYTES, stream);
}
