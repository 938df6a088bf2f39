// Tree-verify attention: every tree node's query attends the left-padded
// prefix KV cache plus the tree's own KV under the ancestor mask.
//
// Sources: EAGLE-Pangu (gist.science ko summary, section 2 Methodology: the
// teacher verifies all speculative tokens in one batched forward with a 4D
// tree mask, node u seeing node v only when v is an ancestor of u; fused
// attention is the performance mode); the nl summary, section 2.C.  Left
// padding of the prefix: Batch Speculative Decoding Done Right (ko summary,
// section 2, rectangular alignment).
//
// The G = Hq/Hkv query heads of a KV head g of sequence b give R = G*T query
// rows r = hl*T + i (hl < G, node i < T) that all read the same keys, so
// Q K^T and P V are dense contractions (bf16 MFMA).  Rows are cut into 16-row
// query tiles.  Two decompositions compute the same function:
//   * stream form (attn_bf16_stream_kernel + attn_stream_combine_kernel): the
//     64-key tiles of all (sequence, KV head, query block) units form one
//     stream cut into one range of equal cost per CU; compute waves own one
//     query tile each, two producer waves stream K and V tiles HBM -> LDS;
//     units cut by range ends leave (m, l, O) partials merged in stream order.
//   * split form (attn_bf16_kernel + attn_combine_kernel): one workgroup per
//     (sequence, KV head, query block, prefix split of kc keys); the last split
//     also takes the tree keys; splits are merged in split order.
// Both are bitwise reproducible for identical inputs.  Tree tile t of a row
// uses its mask word t; masked keys get probability 0 exactly.
//
// bf16 math, per 64-key tile: S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = 16
// keys x 32 dims, one 16-byte LDS read per lane; B = the wave's Q fragment in
// registers), so a lane holds 16 scores of one query row.  Online softmax in
// fp32, base 2.  O^T += V^T P^T: P (rounded to bf16) is already in the B
// operand layout, and V^T comes from LDS with ds_read_b64_tr_b16.  Tiles land
// in LDS unpadded, XOR-swizzled against bank conflicts, by global_load_lds
// copies issued as inline assembly (waits are explicit).
//
// fp32 path: the split structure with VALU arithmetic (one lane per key for
// Q K^T, one lane per dimension for P V).
#include <type_traits>

#include "svt_internal.h"

namespace svt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();
constexpr int KT = 64;  // keys per LDS tile
constexpr float kRescale = 8.0f;  // lazy-rescale threshold, base-2 units

// Stream form: what the combine needs about the unit that range c's last
// piece belongs to, when range c is the first of several ranges holding that
// unit's tiles (the main kernel's workgroup for range c writes it).
struct RangeMeta {
  int u;    // the unit (b * Hkv * nqb + g * nqb + qb), or -1: no unit starts a cut in range c
  int c1;   // last range holding tiles of the unit
  int ntl;  // key tiles of the unit
  int pad0;
  int64_t cu;     // cost position of the unit's set-up
  int64_t p;      // stream position of the unit's first tile
  int64_t ct;     // total cost of the stream
  int64_t pad;
};

struct AttnDev {
  const void* q;
  const void* kcache;
  const void* vcache;
  const void* ktree;
  const void* vtree;
  const uint64_t* mask;
  const int32_t* len;
  const int32_t* lmax;
  const int32_t* status;
  const int32_t* slot;  // sequence -> cache row of k/v_cache, or NULL (identity)
  void* out;
  int32_t* seq_status;
  float* ws_o;   // split form: partials [B][Hkv][ns][R][D]
  float* ws_ml;  // split form: matching (m, l) pairs
  _Float16* ws_h;  // stream form: partial O / l per row, divided by the row's scale s, [2*grid][qb_rows][D]
  float4* ws_mls;  // stream form: (m, l, s, 0) per partial row
  int* ws_pref;  // stream form: tiles before each sequence [B + 1], then non-empty sequences before it [B + 1]
  RangeMeta* ws_meta;  // stream form: one per range
  int64_t cap;
  int B, T, Hq, Hkv, G, R, W;
  int lmax_bound, kc, ns, nqb, qb_rows, nunits;
  int nwk;          // split form: waves sharing each query tile's rows (each takes one 32-key half of every tile)
  int n_slots;      // cache rows when slot is set
  int stream_grid;  // stream form: ranges of the cut (one per CU, or a whole number per unit)
  int rpu;          // stream form: ranges per unit when the grid is a whole number of them per unit, else 0
  int nqt;          // 16-row query tiles per KV head
  int piece_cost;   // stream form: key tiles' worth of time one unit's set-up and output cost
  float scale_log2;
};

// Stream form: query block qb of a KV head holds query tiles
// [unit_tile_lo(qb), unit_tile_lo(qb + 1)); the nqb blocks split the nqt tiles
// as evenly as whole tiles allow.
__device__ __forceinline__ int unit_tile_lo(const AttnDev& a, int qb) { return (int)(((int64_t)qb * a.nqt) / a.nqb); }

// Why sequence b is skipped (SVT_OK: it is not): its tree status, a cache
// row outside the pool, or lengths outside 0 <= len <= lmax <= lmax_bound.
__device__ __forceinline__ int seq_code(const AttnDev& a, int b, int lmax, int L) {
  // the optional arrays are read through a pointer that is never null (len
  // when they are absent), so the loads need no branch and go out together
  // with the lengths'
  const int st0 = (a.status ? a.status : a.len)[b];
  const int row0 = (a.slot ? a.slot : a.len)[b];
  const int st = a.status ? st0 : SVT_OK;
  const int row = a.slot ? row0 : b;
  if (st != SVT_OK) return st;
  if (row < 0 || row >= a.n_slots) return SVT_ERR_ARG;
  return (lmax >= 0 && lmax <= a.lmax_bound && L >= 0 && L <= lmax) ? SVT_OK : SVT_ERR_LENGTH;
}

// Decoded workgroup coordinates and the sequence's key ranges.
struct WgCtx {
  int b, g, split, qb;
  int64_t cg;      // cache slab (cache row * Hkv + g)
  int code;        // SVT_OK or why the sequence is skipped
  int L, lmax;
  int ns_b;        // splits this sequence uses
  int k_beg, k_end;
  int n_ptiles, n_ttiles;
};

// Workgroup coordinates, from the workgroup id alone (no memory access).
__device__ __forceinline__ bool decode_coords(const AttnDev& a, WgCtx& c) {
  // A unit is one (split, sequence, KV head); units are numbered with the
  // split slowest, so the full-size first splits are dispatched before the
  // ragged last ones.  The hardware sends workgroup id w to XCD w % 8: the
  // nqb query blocks of a unit get ids 8 apart, so they run on one XCD and
  // share its L2, while consecutive units spread over all XCDs.
  const int w = blockIdx.x;
  const int span = 8 * a.nqb;
  const int x = w % 8;
  const int unit = (w / span) * 8 + x;
  if (unit >= a.nunits) return false;
  c.qb = (w % span) / 8;
  c.g = unit % a.Hkv;
  c.b = (unit / a.Hkv) % a.B;
  c.split = unit / (a.Hkv * a.B);
  return true;
}

// The sequence's lengths and status, and the key ranges of this split;
// false when the sequence uses fewer splits.
__device__ __forceinline__ bool decode_lengths(const AttnDev& a, WgCtx& c) {
  c.lmax = *a.lmax;
  c.L = a.len[c.b];
  c.code = seq_code(a, c.b, c.lmax, c.L);
  const int row_v = (a.slot ? a.slot : a.len)[c.b];  // the load seq_code made
  c.cg = (int64_t)(c.code == SVT_OK ? (a.slot ? row_v : c.b) : 0) * a.Hkv + c.g;
  c.ns_b = c.code == SVT_OK ? max(1, (c.L + a.kc - 1) / a.kc) : 1;
  if (c.split >= c.ns_b) return false;
  c.k_beg = c.split * a.kc;
  c.k_end = c.code == SVT_OK ? min(c.L, c.k_beg + a.kc) : c.k_beg;
  c.n_ptiles = c.k_end > c.k_beg ? (c.k_end - c.k_beg + KT - 1) / KT : 0;
  c.n_ttiles = (c.split == c.ns_b - 1) ? (a.T + KT - 1) / KT : 0;
  return true;
}

template <typename E>
__device__ void write_zero_rows(const AttnDev& a, const WgCtx& c, int D) {
  // Skipped sequence: split 0 writes zeros over the rows of its query block.
  E* out = static_cast<E*>(a.out);
  const int r0 = c.qb * a.qb_rows;
  const int r1 = min(a.R, r0 + a.qb_rows);
  for (int x = threadIdx.x; x < (r1 - r0) * D; x += blockDim.x) {
    const int r = r0 + x / D, d = x % D;
    const int hl = r / a.T, i = r % a.T;
    out[(((int64_t)c.b * a.T + i) * a.Hq + c.g * a.G + hl) * D + d] = E(0.0f);
  }
}

__device__ __forceinline__ void write_seq_status(const AttnDev& a, const WgCtx& c) {
  if (a.seq_status && c.split == 0 && c.qb == 0 && c.g == 0 && threadIdx.x == 0) a.seq_status[c.b] = c.code;
}

// Wait until at most N of this wave's vector-memory operations are pending.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// --------------------------------------------------------------------------
// bf16 MFMA kernel
// --------------------------------------------------------------------------
// One pipeline stage holds a K tile and a V tile, KT rows of D bf16 each, with
// no padding.  Row r keeps its 16-byte chunk c at slot c ^ swz(r); the swizzles
// spread the rows that one operand read touches over all 64 LDS banks (K: 16
// rows x one chunk per ds_read_b128; V: 8 rows x two chunks x two halves per
// 32 lanes of ds_read_b64_tr_b16).  Tiles are copied straight from HBM to LDS
// with global_load_lds_dwordx4: one wave instruction fills 1 KB of LDS (64
// lanes x 16 B, consecutive), so the swizzle is applied on the global side by
// choosing which chunk each lane fetches.  No tile data passes through
// registers, and kStages - 1 tiles are in flight while one is computed on.
template <int D, int NW>
struct Tile {
  static constexpr int ROWB = D * 2;
  static constexpr int CPR = ROWB / 16;       // 16-byte chunks per row
  static constexpr int TILEB = KT * ROWB;     // one K or V tile
  static constexpr int STAGEB = 2 * TILEB;
  static constexpr int NINSTR = TILEB / 1024;  // 1 KB copy instructions per K or V tile
  static constexpr int PER_WAVE = (NINSTR + NW - 1) / NW;  // per wave (NW waves share a tile)
  static constexpr int RPI = 1024 / ROWB;      // rows per copy instruction
  // Copy j of wave w is block w + NW * j; when NW does not divide NINSTR the
  // last round has fewer blocks than waves and the waves past them skip it.
  static constexpr bool EXACT = NINSTR % NW == 0;
  __device__ static __forceinline__ bool has_copy(int w, int j) { return EXACT || w + NW * j < NINSTR; }
  // Waits until at most `later` tiles' copies of this wave are pending; a wave
  // that skips the last round has 2 * (PER_WAVE - 1) copies per tile.
  template <int LATER>
  __device__ static __forceinline__ void wait_tiles(int w) {
    if (has_copy(w, PER_WAVE - 1)) wait_vmcnt<2 * PER_WAVE * LATER>();
    else wait_vmcnt<2 * (PER_WAVE - 1) * LATER>();
  }
  __device__ static __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static __forceinline__ int swz_v(int r) { return D == 128 ? ((r & 7) << 1) : (((r >> 1) & 3) << 1); }
};

constexpr int kMaxQbRows = 256;  // query rows per workgroup
typedef __attribute__((address_space(3))) void lds_void;

// 16-byte copy global -> LDS (global_load_lds_dwordx4): lane i's 16 bytes land
// at LDS address lds + 16 * i, with `lds` the same for the whole wave (it goes
// to M0).  Issued as inline assembly on purpose: the compiler would otherwise
// track these copies and wait for all of them (vmcnt(0)) before every use of
// LDS data, which serialises the prefetch with the compute.  Completion is
// tracked by hand with wait_vmcnt<N>() before the workgroup barrier.  M0 is
// not used for anything else in the kernels of this file.
__device__ __forceinline__ void copy16_to_lds(const void* g, unsigned char* lds) {
  const uint32_t la = (uint32_t)(uintptr_t)(lds_void*)lds;
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(la) : "memory");
}

// Makes the compiler complete the loads of x here.  Its wait-count pass does
// not see the asm copies; a register loaded before the main loop and first
// read inside it would otherwise get a vmcnt(0) wait inside the loop, which
// also waits for every prefetched tile.
template <typename V>
__device__ __forceinline__ void settle(const V& x) { asm volatile("" ::"v"(x)); }

// Workgroup barrier that does not wait for outstanding global loads (the
// copies of later tiles stay in flight); pending LDS reads are drained first.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Reductions over the four 16-lane groups of a wave (lanes l, l^16, l^32,
// l^48) with the gfx950 lane-swap instructions.  With both operands equal to
// x, the two results of a swap are x at lane l and at its partner, in some
// order, so a symmetric combine of them gives the pairwise reduction.
__device__ __forceinline__ float group_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// NST: depth of the LDS ring (2: one tile in flight, two workgroups fit per CU;
// 4: three tiles in flight, one workgroup per CU).
// NW: waves per workgroup (3 or 4).
template <int D, int QW, int NST, int NW>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(AttnDev a) {
  constexpr int kStages = NST;
  constexpr int NKS = D / 32;  // 32-wide k steps over the head dim
  constexpr int NDT = D / 16;  // 16-wide output dim tiles
  using TL = Tile<D, NW>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kStages * TL::STAGEB];
  __shared__ uint64_t maskw[kMaxQbRows * 4];

  WgCtx c;
  if (!decode_coords(a, c)) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps wave branches scalar
  const int lane = tid & 63;
  const int n16 = lane & 15;  // row/col inside a 16x16 tile
  const int grp = lane >> 4;  // lane group 0..3
  const int nwk = a.nwk;  // 2: a pair of waves shares the rows, one 32-key half of every tile each
  const int wq = wave / nwk, wk = wave % nwk;

  const uint16_t* __restrict__ q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ kc = static_cast<const uint16_t*>(a.kcache);
  const uint16_t* __restrict__ vc = static_cast<const uint16_t*>(a.vcache);
  const uint16_t* __restrict__ ktr = static_cast<const uint16_t*>(a.ktree);
  const uint16_t* __restrict__ vtr = static_cast<const uint16_t*>(a.vtree);
  const int64_t bg = (int64_t)c.b * a.Hkv + c.g;
  const int r0 = c.qb * a.qb_rows;

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds query row n16 of
  // each of its tiles, dims ks*32 + 8*grp .. +7.  Their addresses need no
  // lengths, so they are requested before the lengths are read.
  bf16x8 qf[QW][NKS];
  int row_node[QW];  // node index of this lane's query row, -1 if padding
  int row_head[QW];
#pragma unroll
  for (int t = 0; t < QW; ++t) {
    const int r = r0 + (wq * QW + t) * 16 + n16;
    const bool ok = r < a.R;
    row_node[t] = ok ? r % a.T : -1;
    row_head[t] = ok ? c.g * a.G + r / a.T : 0;
    const uint16_t* qrow = q + (((int64_t)c.b * a.T + (ok ? row_node[t] : 0)) * a.Hq + row_head[t]) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (ok) {
        qf[t][ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 32 + grp * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[t][ks][e] = (__bf16)0.0f;
      }
    }
  }

  if (!decode_lengths(a, c)) return;
  write_seq_status(a, c);
  if (c.code != SVT_OK) {
    if (c.split == 0) write_zero_rows<__bf16>(a, c, D);
    return;
  }

  const int n_tiles = c.n_ptiles + c.n_ttiles;
  const int pad = c.lmax - c.L;

  auto tile_rows = [&](int t, const uint16_t*& kb, const uint16_t*& vb, int& nvalid) {
    if (t < c.n_ptiles) {
      const int k0 = c.k_beg + t * KT;
      const int64_t col = (int64_t)pad + k0;
      kb = kc + (c.cg * a.cap + col) * D;
      vb = vc + (c.cg * a.cap + col) * D;
      nvalid = min(KT, c.k_end - k0);
    } else {
      const int j0 = (t - c.n_ptiles) * KT;
      kb = ktr + (bg * a.T + j0) * D;
      vb = vtr + (bg * a.T + j0) * D;
      nvalid = min(KT, a.T - j0);
    }
  };
  // Copy tile t into stage `st`: 1 KB blocks dealt round-robin to the waves
  // (a wave past the last block of the final round skips it and waits on
  // its own smaller count).  Rows past the valid ones repeat the last valid
  // row; they are masked out.
  // Per-lane source rows and swizzled chunk offsets of this wave's copies.
  int crow[TL::PER_WAVE], ck[TL::PER_WAVE], cv[TL::PER_WAVE];
#pragma unroll
  for (int j = 0; j < TL::PER_WAVE; ++j) {
    const int row = ((wave + NW * j) % TL::NINSTR) * TL::RPI + lane / TL::CPR;
    const int slot = lane % TL::CPR;
    crow[j] = row;
    ck[j] = 8 * (slot ^ TL::swz_k(row));
    cv[j] = 8 * (slot ^ TL::swz_v(row));
  }
  auto issue_tile = [&](int t, int st) {
    const uint16_t *kb, *vb;
    int nvalid;
    tile_rows(t, kb, vb, nvalid);
    unsigned char* kl = lds + st * TL::STAGEB;
    unsigned char* vl = kl + TL::TILEB;
#pragma unroll
    for (int j = 0; j < TL::PER_WAVE; ++j) {
      if (!TL::has_copy(wave, j)) continue;
      const int ins = (wave + NW * j) % TL::NINSTR;
      const int src = (nvalid == KT ? crow[j] : min(crow[j], nvalid - 1)) * D;
      copy16_to_lds(kb + src + ck[j], kl + ins * 1024);
      copy16_to_lds(vb + src + cv[j], vl + ins * 1024);
    }
  };

  // The first tiles' copies travel with the Q fragments (the wait for Q
  // below also covers them: completion is counted in issue order).
#pragma unroll
  for (int st = 0; st < kStages - 1; ++st)
    if (st < n_tiles) issue_tile(st, st);

  bool tile_live[QW];  // does the tile hold any real row?  (wave-uniform)
#pragma unroll
  for (int t = 0; t < QW; ++t) tile_live[t] = r0 + (wq * QW + t) * 16 < a.R;
  // Waves with a real row compute all QW tiles (padding rows have Q = 0 and
  // are never stored), so the MFMA chains need no per-tile branches.
  const bool wave_live = __builtin_amdgcn_readfirstlane(tile_live[0] ? 1 : 0) != 0;
#pragma unroll
  for (int t = 0; t < QW; ++t)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) settle(qf[t][ks]);

  // Ancestor-mask words of the block's rows, for the tree tiles.
  if (c.n_ttiles > 0) {
    for (int x = tid; x < a.qb_rows * a.W; x += NW * 64) {
      const int rl = x / a.W, w = x % a.W, r = r0 + rl;
      maskw[rl * 4 + w] = r < a.R ? a.mask[((int64_t)c.b * a.T + r % a.T) * a.W + w] : 0ull;
    }
  }
  __syncthreads();

  // Online softmax state per query row, in base-2 units of scale * q.k.
  // m_ref is the reference the accumulators are scaled to; it moves (and O,
  // l are rescaled) only when a score exceeds it by more than kRescale, which
  // happens in the first tiles and then rarely.  O / l does not depend on it.
  // Padding rows (Q = 0, so every score is exactly 0) start at m_ref = 0 and
  // never trigger a rescale; their accumulators are never stored.
  // l is accumulated by the matrix cores: one extra MFMA per 32 keys with an
  // all-ones A operand sums the bf16 P exactly as the P V product uses it, and
  // leaves the row sum in every element of the lane's accumulator.
  f32x4 o[QW][NDT];
  f32x4 lacc[QW];
  float m_ref[QW];
#pragma unroll
  for (int t = 0; t < QW; ++t) {
    m_ref[t] = row_node[t] >= 0 ? kNegInf : 0.0f;
    lacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
  const float sc = a.scale_log2;

  // Lane-constant LDS byte offsets.  Sub-tiles start at multiples of 16 keys
  // (K) and 32 keys (V), so every swizzle depends on the lane alone.
  int koff[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) koff[ks] = n16 * TL::ROWB + 16 * ((ks * 4 + grp) ^ TL::swz_k(n16));
  const int vrow = 4 * grp + (n16 >> 2);  // + kb0, and + 16 for the second read
  const int q4 = lane & 3;
  int voff[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
    voff[dt] = vrow * TL::ROWB + 16 * ((2 * dt + (q4 >> 1)) ^ TL::swz_v(vrow)) + 8 * (q4 & 1);

  // One 32-key half of the current tile.  MASKED selects the path with
  // per-key validity bits (ragged tail, tree tiles); full prefix halves skip it.
  auto process_half = [&](auto masked_c, const unsigned char* kl, const unsigned char* vl, int kb0,
                          const uint64_t* vbits) {
    constexpr bool MASKED = decltype(masked_c)::value;
    // S^T = K Q^T: A operand rows = keys kb0 + 16u + n16, dims ks*32 + 8*grp.
    // All QW x 2 accumulation chains are advanced together so that
    // consecutive MFMAs are independent.
    const unsigned char* kh = kl + kb0 * TL::ROWB;
    bf16x8 kf[2][NKS];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        kf[u][ks] = *reinterpret_cast<const bf16x8*>(kh + 16 * u * TL::ROWB + koff[ks]);
    // V^T fragments (transposing LDS reads) are requested now, so that their
    // latency overlaps the score MFMAs and the softmax.  Lane (lambda)
    // addresses key kb0 + 4*(lambda/16) + (lambda%16)/4 (+16), dims
    // dt*16 + 4*(lambda%4).
    const unsigned char* vh = vl + kb0 * TL::ROWB;
    bf16x8 vf[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vh + voff[dt]));
      const s16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vh + 16 * TL::ROWB + voff[dt]));
      vf[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    f32x4 s[QW][2];
#pragma unroll
    for (int qt = 0; qt < QW; ++qt)
#pragma unroll
      for (int u = 0; u < 2; ++u) s[qt][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int qt = 0; qt < QW; ++qt)
          s[qt][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[u][ks], qf[qt][ks], s[qt][u], 0, 0, 0);
    bf16x8 pf[QW];
#pragma unroll
    for (int qt = 0; qt < QW; ++qt) {
      // lane holds raw scores of query n16 for keys kb0 + 16u + 4*grp + e
      float x[8];
      uint32_t bits = 0;
      if constexpr (MASKED) bits = (uint32_t)(vbits[qt] >> (kb0 + 4 * grp));
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = s[qt][u][e];
          if constexpr (MASKED) v = ((bits >> (16 * u + e)) & 1u) ? v : kNegInf;
          x[u * 4 + e] = v;
        }
      float lmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
      lmax *= sc;  // sc > 0: the max of scaled scores
      if (__any(lmax > m_ref[qt] + kRescale)) {  // wave-uniform; first tiles, then rare
        // only the rows over their own threshold move their reference, so a
        // row's result never depends on another row's scores
        const float m_new = fmaxf(m_ref[qt], group_max(lmax));
        if (m_new > m_ref[qt] + kRescale || m_ref[qt] == kNegInf) {
          const float alpha = m_new == kNegInf ? 1.0f : __builtin_amdgcn_exp2f(m_ref[qt] - m_new);
          lacc[qt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[qt][dt] *= alpha;
          m_ref[qt] = m_new;
        }
      }
      const float neg_m = m_ref[qt] == kNegInf ? 0.0f : -m_ref[qt];
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[qt][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(x[e], sc, neg_m));
    }
    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int qt = 0; qt < QW; ++qt)
        o[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pf[qt], o[qt][dt], 0, 0, 0);
#pragma unroll
    for (int qt = 0; qt < QW; ++qt)
      lacc[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[qt], lacc[qt], 0, 0, 0);
  };



  for (int t = 0; t < n_tiles; ++t) {
    // tile t has landed once at most the copies of later tiles are pending
    static_assert(kStages == 2 || kStages == 4, "wait ladder covers 2 or 4 stages");
    const int later = min(kStages - 2, n_tiles - 1 - t);
    if (kStages == 4 && later >= 2) TL::template wait_tiles<2>(wave);
    else if (kStages == 4 && later == 1) TL::template wait_tiles<1>(wave);
    else wait_vmcnt<0>();
    lds_barrier();
    if (t + kStages - 1 < n_tiles) issue_tile(t + kStages - 1, (t + kStages - 1) % kStages);

    const bool tree_tile = t >= c.n_ptiles;
    int nvalid;
    {
      const uint16_t *kb_, *vb_;
      tile_rows(t, kb_, vb_, nvalid);
    }
    const unsigned char* kl = lds + (t % kStages) * TL::STAGEB;
    const unsigned char* vl = kl + TL::TILEB;
    if (!wave_live) {
      // no real query row in this wave: it only helps with the copies
    } else if (!tree_tile && nvalid == KT) {
#pragma unroll 1
      for (int half = 0; half < 2; ++half) {
        if (nwk == 2 && half != wk) continue;
        process_half(std::false_type{}, kl, vl, half * 32, nullptr);
      }
    } else {
      // Valid-key bits of this tile per query row: the first nvalid keys, and
      // for tree tiles only the ancestors.
      const uint64_t head_bits = nvalid >= 64 ? ~0ull : ((1ull << nvalid) - 1ull);
      uint64_t vbits[QW];
#pragma unroll
      for (int qt = 0; qt < QW; ++qt) {
        uint64_t v = row_node[qt] >= 0 ? head_bits : 0ull;
        if (tree_tile) v &= maskw[((wq * QW + qt) * 16 + n16) * 4 + (t - c.n_ptiles)];
        vbits[qt] = v;
      }
#pragma unroll 1
      for (int half = 0; half < 2; ++half) {
        if (nwk == 2 && half != wk) continue;
        if (half * 32 >= nvalid) continue;  // wave-uniform: nothing valid in this half
        process_half(std::true_type{}, kl, vl, half * 32, vbits);
      }
    }
  }
  lds_barrier();  // every wave is done with the stage buffers

  // ---- two waves that split key tiles merge their states through LDS
  float* xo = reinterpret_cast<float*>(lds);
  if (nwk == 2) {
    constexpr int PER_LANE = QW * NDT * 4 + 2 * QW;
    float* slot = xo + (wq * 64 + lane) * PER_LANE;
    if (wk == 1) {
      int k = 0;
#pragma unroll
      for (int qt = 0; qt < QW; ++qt) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int e = 0; e < 4; ++e) slot[k++] = o[qt][dt][e];
        slot[k++] = m_ref[qt];
        slot[k++] = lacc[qt][0];
      }
    }
    __syncthreads();
    if (wk == 1) return;
    int k = 0;
#pragma unroll
    for (int qt = 0; qt < QW; ++qt) {
      f32x4 o1[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) o1[dt][e] = slot[k++];
      const float m1 = slot[k++];
      const float l1 = slot[k++];
      const float mm = fmaxf(m_ref[qt], m1);
      const float a0 = mm == kNegInf ? 1.0f : exp2f(m_ref[qt] - mm);
      const float a1 = mm == kNegInf ? 1.0f : exp2f(m1 - mm);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[qt][dt] = o[qt][dt] * a0 + o1[dt] * a1;
      lacc[qt][0] = lacc[qt][0] * a0 + l1 * a1;
      m_ref[qt] = mm;
    }
  }

  // ---- epilogue: lane holds O^T[d = dt*16 + 4*grp + e][query n16]
  const bool direct = c.ns_b == 1;
#pragma unroll
  for (int qt = 0; qt < QW; ++qt) {
    if (!tile_live[qt]) continue;
    const float lt = lacc[qt][0];
    if (row_node[qt] < 0) continue;
    const int r = r0 + (wq * QW + qt) * 16 + n16;
    if (direct) {
      const float inv = 1.0f / lt;
      __bf16* orow = static_cast<__bf16*>(a.out) + (((int64_t)c.b * a.T + row_node[qt]) * a.Hq + row_head[qt]) * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[qt][dt][e] * inv);
        *reinterpret_cast<bf16x4*>(orow + dt * 16 + 4 * grp) = v;
      }
    } else {
      const int64_t pr = ((bg * a.ns + c.split) * a.R + r);
      float* po = a.ws_o + pr * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4*>(po + dt * 16 + 4 * grp) = o[qt][dt];
      if (grp == 0) {
        a.ws_ml[pr * 2 + 0] = m_ref[qt];
        a.ws_ml[pr * 2 + 1] = lt;
      }
    }
  }
}

// --------------------------------------------------------------------------
// bf16 MFMA kernel, stream form (used when the batch gives every CU eight or
// more key tiles).  A work unit is one (sequence, KV head, query block): up to 12
// query tiles of 16 rows, one per compute wave, so every K/V tile of the unit
// crosses HBM -> LDS once and feeds all of its query rows.  A unit's key tiles
// are its prefix tiles followed by its tree tiles; the tiles of all units,
// concatenated in unit order, form one stream that is cut into gridDim.x
// ranges of equal cost (tiles plus a set-up cost per unit), one per workgroup
// (one workgroup per CU).  A workgroup walks its
// range with one 4-deep DMA ring that runs across unit boundaries, fed by two
// producer waves (one copies the K planes, the other the V planes) that do no
// arithmetic: copies that stall on issue under memory back-pressure never hold
// up a compute wave, and the compute waves' own loads (Q, mask words) never
// wait behind tile copies.  A unit lying wholly inside
// one range is normalised and written directly; a unit cut by range ends
// leaves (m, l, O) partials in two slots per range c (slot 2c + 1: the
// range's last piece when its unit goes on past the range end; slot 2c: the
// range's first piece when it continues a unit from an earlier range and
// ends with it), and attn_stream_combine_kernel merges them in stream order.  No workgroup waits
// for another, and the result does not depend on timing.
// --------------------------------------------------------------------------
constexpr int kStreamMaxB = kStreamMaxBatch;

// Key tiles one unit of sequence b holds (prefix tiles + tree tiles), or 0
// when the sequence is skipped; *code says why.
__device__ __forceinline__ int stream_seq_tiles(const AttnDev& a, int b, int lmax, int* code) {
  const int L = a.len[b];
  *code = seq_code(a, b, lmax, L);
  return *code == SVT_OK ? (L + KT - 1) / KT + (a.T + KT - 1) / KT : 0;
}

// floor(a / b) for 0 <= a < 2^53 and 0 < b < 2^53: the double quotient is
// within one of it (relative error below 2^-53), one integer step corrects
// it.  Cheaper than the 64-bit integer division, which is a long software
// sequence on the GPU.
__device__ __forceinline__ int64_t div_floor(int64_t a, int64_t b) {
  int64_t q = (int64_t)((double)a / (double)b);
  if (q * b > a) --q;
  else if ((q + 1) * b <= a) ++q;
  return q;
}
// Stream position of the first tile of workgroup range c (ranges are floor(c*N/G)).
__device__ __forceinline__ int64_t stream_lo(int64_t c, int64_t n, int g) { return div_floor(c * n, g); }
// Range holding stream tile x.
__device__ __forceinline__ int stream_range_of(int64_t x, int64_t n, int g) { return (int)div_floor((x + 1) * g - 1, n); }

// The ranges that hold tiles of one unit.  The unit's cost interval is
// [cu, cu + pc + ntl) (its set-up, then its tiles) and its tiles are stream
// tiles [p, p + ntl); the ranges are g equal cuts of the total cost ct, and a
// range boundary at cost q inside the unit's tiles falls before tile
// p + (q - cu - pc).  Ranges c0..c1 touch the unit.
struct UnitCut {
  int64_t ct, cu, p;
  int g, pc, ntl, c0, c1;
};
__device__ __forceinline__ UnitCut unit_cut(int64_t ct, int64_t cu, int64_t p, int g, int pc, int ntl) {
  UnitCut u{ct, cu, p, g, pc, ntl, 0, 0};
  u.c0 = stream_range_of(cu + pc, ct, g);
  u.c1 = stream_range_of(cu + pc + ntl - 1, ct, g);
  return u;
}
// Whether range cc (c0 <= cc <= c1) holds a piece of the unit (ranges between
// c0 and c1 may be empty when there are fewer tiles than ranges), and the
// partial slot that piece leaves: 2cc + 1 when the unit goes on past the
// range (cc < c1), 2cc for its last piece (range c1).
__device__ __forceinline__ bool unit_piece(const UnitCut& u, int cc, int* slot) {
  const int64_t clo = stream_lo(cc, u.ct, u.g), chi = stream_lo(cc + 1, u.ct, u.g);
  const int64_t tlo = cc == u.c0 ? u.p : u.p + (clo - u.cu - u.pc);
  const int64_t thi = cc < u.c1 ? u.p + (chi - u.cu - u.pc) : u.p + u.ntl;
  *slot = 2 * cc + (cc < u.c1 ? 1 : 0);
  return tlo < thi;
}

// One step of the in-order merge of a row's pieces: (mx, l, acc) holds the
// merged maximum (base 2), weight and output of the pieces so far; the piece
// brings its maximum mj, its weight lj, its output divided by lj and by its
// scale sj (oi) and that scale.  A piece that sees no key of the row has
// mj = -inf and is skipped.
template <int N>
__device__ __forceinline__ void merge_piece(float& mx, float& l, float (&acc)[N], float mj, float lj, float sj,
                                            const float (&oi)[N]) {
  if (mj == kNegInf) return;
  const float mn = fmaxf(mx, mj);
  const float s0 = exp2f(mx - mn), s1 = exp2f(mj - mn);
  const float w = lj * s1;  // weight of the piece's normalised output
  const float ws = w * sj;  // times its scale
  l = l * s0 + w;
#pragma unroll
  for (int e = 0; e < N; ++e) acc[e] = acc[e] * s0 + oi[e] * ws;
  mx = mn;
}

// NW compute waves (QMAX query tiles each) and two producer waves.
template <int D, int NW, int QMAX>
__global__ __launch_bounds__((NW + 2) * 64) void attn_bf16_stream_kernel(AttnDev a) {
  constexpr int NP = 2;  // producer waves: K planes, V planes
  constexpr int kStages = 4;
  constexpr int NKS = D / 32;
  constexpr int NDT = D / 16;
  constexpr int NT = (NW + NP) * 64;
  using TL = Tile<D, NW>;
  static_assert(3 * TL::NINSTR < 64, "a producer's three tiles in flight must fit its vmcnt range");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kStages * TL::STAGEB];
  __shared__ int s_pref[kStreamMaxB + 1];  // s_pref[b] = tiles of sequences < b (per unit)
  __shared__ int s_len[kStreamMaxB];
  __shared__ int s_row[kStreamMaxB];  // cache row of each sequence
  __shared__ int s_npref[kStreamMaxB + 1];  // non-empty sequences before b
  __shared__ int s_wsum[NW + NP], s_wsum2[NW + NP];
  __shared__ int s_carry, s_carry2;
  __shared__ uint64_t s_mask[NW * QMAX * 16][4];  // each lane's tree-mask words, its own rows only

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n16 = lane & 15;
  const int grp = lane >> 4;
  const int B = a.B;
  const int lmax = *a.lmax;
  // With nine or twelve compute waves, waves 4..7 run each tile half a step
  // behind the others (see run_piece): waves w, w + 4, w + 8 share a SIMD, so
  // every SIMD then holds a lagging and a leading wave whose matrix and
  // vector phases overlap instead of coinciding after every barrier (B=1 32K
  // with twelve: 59.6 -> 56.9 us per call; with eight waves it was slower).
#ifndef SVT_STREAM_LAG
#define SVT_STREAM_LAG 1
#endif
  constexpr bool kLagging = SVT_STREAM_LAG && (NW == 9 || NW == 12);
  const bool lag = kLagging && wave < NW && ((wave >> 2) & 1);

  // ---- per-sequence tile counts and their prefix (every workgroup computes it)
  // With at most 64 sequences every wave holds the table in registers (lane
  // b: sequence b) and finds its range bounds and first unit with wave
  // ballots, so the first copies wait for one round of loads and no barrier;
  // wave 0 also stores the table in LDS for the walk through the range.
  // Larger batches build it in LDS with a workgroup-wide scan.
  const bool small_b = B <= 64;
  int rv = 0, rx = 0, rx2 = 0, rL = 0, rrow = 0;  // small batch, lane b: tiles, inclusive prefixes, length, cache row
  if (small_b) {
    const int b = lane;
    int code;
    if (b < B) {
      rv = stream_seq_tiles(a, b, lmax, &code);
      rL = a.len[b];
      rrow = a.slot ? a.slot[b] : b;
    }
    rx = rv;
    rx2 = rv > 0 ? 1 : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(rx, o), y2 = __shfl_up(rx2, o);
      if (lane >= o) {
        rx += y;
        rx2 += y2;
      }
    }
    if (wave == 0) {
      if (b < B) {
        s_pref[b + 1] = rx;
        s_npref[b + 1] = rx2;
        s_len[b] = rL;
        s_row[b] = rrow;
      }
      if (lane == 0) {
        s_pref[0] = 0;
        s_npref[0] = 0;
      }
    }
  } else {
    if (tid == 0) {
      s_pref[0] = 0;
      s_npref[0] = 0;
      s_carry = 0;
      s_carry2 = 0;
    }
    __syncthreads();
    for (int base = 0; base < B; base += NT) {
      const int b = base + tid;
      int v = 0, code;
      if (b < B) {
        v = stream_seq_tiles(a, b, lmax, &code);
        s_len[b] = a.len[b];
        s_row[b] = a.slot ? a.slot[b] : b;
      }
      int x = v, x2 = v > 0 ? 1 : 0;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o), y2 = __shfl_up(x2, o);
        if (lane >= o) {
          x += y;
          x2 += y2;
        }
      }
      if (lane == 63) {
        s_wsum[wave] = x;
        s_wsum2[wave] = x2;
      }
      __syncthreads();
      int off = s_carry, off2 = s_carry2;
      for (int w = 0; w < wave; ++w) {
        off += s_wsum[w];
        off2 += s_wsum2[w];
      }
      if (b < B) {
        s_pref[b + 1] = off + x;
        s_npref[b + 1] = off2 + x2;
      }
      __syncthreads();
      if (tid == NT - 1) {
        s_carry = off + x;
        s_carry2 = off2 + x2;
      }
      __syncthreads();
    }
  }
  const int G = a.stream_grid;  // ranges of the cut; workgroups past them (if any) get none
  // Consecutive ranges go to one XCD (the hardware sends workgroup w to XCD
  // w % 8), so the query blocks of one KV head, adjacent in the stream, tend
  // to share an L2.
  const int NG = gridDim.x;
  int c = (NG % 8 == 0) ? (int)(blockIdx.x % 8) * (NG / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  if (a.rpu > 0 && c < G) {
    // A whole number of ranges per unit (one sequence): consecutive
    // workgroup slots take the same key range of every query block of a KV
    // head, so the workgroups of one XCD read the same K/V tiles at about the
    // same time and its L2 serves all but the first read of each.
    const int qb = c % a.nqb, r = (c / a.nqb) % a.rpu, g = c / (a.nqb * a.rpu);
    c = (g * a.nqb + qb) * a.rpu + r;
  }
  const int UPB = a.Hkv * a.nqb;  // units per sequence
  // tiles and non-empty sequences of the whole batch
  const int tot_t = small_b ? __builtin_amdgcn_readlane(rx, 63) : s_pref[B];
  const int tot_n = small_b ? __builtin_amdgcn_readlane(rx2, 63) : s_npref[B];
  const int64_t N = (int64_t)UPB * tot_t;
  // Ranges are equal in cost, not in tiles: a unit costs its key tiles plus
  // piece_cost for its set-up and output, so a range that starts several
  // units gets fewer tiles.  Cost position p maps to the stream tile it
  // reaches (positions inside a unit's set-up map to its first tile).
  const int PC = a.piece_cost;
  auto seq_cost = [&](int b) { return (int64_t)UPB * ((int64_t)s_pref[b] + (int64_t)PC * s_npref[b]); };
  const int64_t CT = (int64_t)UPB * ((int64_t)tot_t + (int64_t)PC * tot_n);
  // The last sequence l whose cost, or (by_tile) whose first stream tile, is
  // at most p, with its tiles before it, non-empty sequences before it and
  // tile count; never an empty sequence (the next one starts at the same
  // position).  Small batch: one ballot over the lanes; otherwise a binary
  // search of the LDS table.
  struct SeqAt {
    int l, pref, npref, ntl;
  };
  auto seq_at = [&](int64_t p, bool by_tile) -> SeqAt {
    SeqAt r;
    if (small_b) {
      const int pe = rx - rv, pe2 = rx2 - (rv > 0 ? 1 : 0);  // this lane's exclusive prefixes
      const int64_t key = (int64_t)UPB * (by_tile ? (int64_t)pe : (int64_t)pe + (int64_t)PC * pe2);
      const uint64_t m = __ballot(lane < B && key <= p);  // lane 0 always qualifies (p >= 0)
      r.l = 63 - __builtin_clzll(m);
      r.pref = __builtin_amdgcn_readlane(pe, r.l);
      r.npref = __builtin_amdgcn_readlane(pe2, r.l);
      r.ntl = __builtin_amdgcn_readlane(rv, r.l);
    } else {
      int l = 0, h = B;
      while (h - l > 1) {
        const int m = (l + h) >> 1;
        if ((by_tile ? (int64_t)UPB * s_pref[m] : seq_cost(m)) <= p) l = m;
        else h = m;
      }
      r.l = __builtin_amdgcn_readfirstlane(l);
      r.pref = __builtin_amdgcn_readfirstlane(s_pref[r.l]);
      r.npref = __builtin_amdgcn_readfirstlane(s_npref[r.l]);
      r.ntl = __builtin_amdgcn_readfirstlane(s_pref[r.l + 1]) - r.pref;
    }
    return r;
  };
  auto cost_to_tile = [&](int64_t p) -> int64_t {
    if (p >= CT) return N;
    const SeqAt q = seq_at(p, false);
    const int off = (int)(p - (int64_t)UPB * ((int64_t)q.pref + (int64_t)PC * q.npref));
    const int j = off / (q.ntl + PC), r = off - j * (q.ntl + PC);
    return (int64_t)UPB * q.pref + (int64_t)j * q.ntl + max(0, r - PC);
  };
  const int64_t lo = cost_to_tile(stream_lo(c, CT, G)), hi = cost_to_tile(stream_lo(c + 1, CT, G));
  // The combine's record of this range: when the range ends inside a unit
  // whose first tile it holds, the unit and the ranges of its pieces, so
  // that the combine needs no prefix table to find them.  Wave 0 computes it
  // (the small-batch search is a ballot over its lanes) before its first
  // loads; lane 0 stores it.
  // Not needed when the combine finds the pieces without it: one sequence,
  // a whole number of ranges per unit, every range holding tiles of its unit
  // (the combine's test, on the same numbers).
  const bool need_meta = a.ws_meta && c < G && !(a.rpu > 0 && tot_t > 0 && (tot_t + PC) / a.rpu >= PC + 2);
  auto range_meta = [&]() {
    RangeMeta m{-1, 0, 0, 0, 0, 0, 0, 0};
    if (lo < hi) {
      const SeqAt q = seq_at(hi - 1, true);  // the sequence of the range's last tile
      const int64_t sb = (int64_t)UPB * q.pref;
      const int j = (int)div_floor(hi - 1 - sb, q.ntl);
      const int64_t base = sb + (int64_t)j * q.ntl;
      if (hi < base + q.ntl) {
        const int64_t cu = (int64_t)UPB * ((int64_t)q.pref + (int64_t)PC * q.npref) + (int64_t)j * (q.ntl + PC);
        const UnitCut uc = unit_cut(CT, cu, base, G, PC, q.ntl);
        if (uc.c0 == c && uc.c1 > c) m = RangeMeta{q.l * UPB + j, uc.c1, q.ntl, 0, cu, base, CT, 0};
      }
    }
    return m;
  };
  if (wave == 0 && need_meta) {
    const RangeMeta m = range_meta();
    if (lane == 0) a.ws_meta[c] = m;
  }

  const uint16_t* __restrict__ q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ kc = static_cast<const uint16_t*>(a.kcache);
  const uint16_t* __restrict__ vc = static_cast<const uint16_t*>(a.vcache);
  const uint16_t* __restrict__ ktr = static_cast<const uint16_t*>(a.ktree);
  const uint16_t* __restrict__ vtr = static_cast<const uint16_t*>(a.vtree);

  // Cursor over the stream: unit (b, j = g*nqb + qb), its first tile `base`,
  // its tile count, and what the per-tile source addresses need (content
  // length, prefix tiles, base pointers), refreshed only when the cursor
  // enters a unit.  All fields are wave-uniform.
  struct Cur {
    int b, j, ntl, L, np;
    int64_t base;
    const uint16_t *kp, *vp, *kt, *vt;  // prefix content start, tree rows
  };
  auto fill_lr = [&](Cur& r, int L, int row) {
    r.L = L;
    r.np = (r.L + KT - 1) / KT;
    const int64_t bg = (int64_t)r.b * a.Hkv + r.j / a.nqb;
    const int64_t cg = (int64_t)row * a.Hkv + r.j / a.nqb;
    r.kp = kc + (cg * a.cap + (lmax - r.L)) * D;
    r.vp = vc + (cg * a.cap + (lmax - r.L)) * D;
    r.kt = ktr + bg * a.T * D;
    r.vt = vtr + bg * a.T * D;
  };
  auto fill = [&](Cur& r) {
    fill_lr(r, __builtin_amdgcn_readfirstlane(s_len[r.b]), __builtin_amdgcn_readfirstlane(s_row[r.b]));
  };
  // The unit holding stream tile x (small batch: the sequence's length and
  // cache row come from the lanes, not from LDS).
  auto locate = [&](int64_t x) {
    const SeqAt q = seq_at(x, true);
    Cur r;
    r.b = q.l;
    r.ntl = q.ntl;
    const int64_t sb = (int64_t)UPB * q.pref;
    r.j = (int)div_floor(x - sb, r.ntl);
    r.base = sb + (int64_t)r.j * r.ntl;
    if (small_b) fill_lr(r, __builtin_amdgcn_readlane(rL, r.b), __builtin_amdgcn_readlane(rrow, r.b));
    else fill(r);
    return r;
  };
  auto advance = [&](Cur& r) {
    r.base += r.ntl;
    if (++r.j == UPB) {
      r.j = 0;
      do {
        ++r.b;
      } while (r.b < B && s_pref[r.b + 1] == s_pref[r.b]);
      r.ntl = r.b < B ? __builtin_amdgcn_readfirstlane(s_pref[r.b + 1] - s_pref[r.b]) : 0;
    }
    if (r.b < B) fill(r);
  };

  // Source rows of stream tile x of unit `r`; tree_t = -1 for a prefix tile.
  auto tile_src = [&](const Cur& r, int64_t x, const uint16_t*& kb, const uint16_t*& vb, int& nvalid, int& tree_t) {
    const int t = (int)(x - r.base);
    if (t < r.np) {
      kb = r.kp + (int64_t)t * (KT * D);
      vb = r.vp + (int64_t)t * (KT * D);
      nvalid = min(KT, r.L - t * KT);
      tree_t = -1;
    } else {
      const int j0 = (t - r.np) * KT;
      kb = r.kt + (int64_t)j0 * D;
      vb = r.vt + (int64_t)j0 * D;
      nvalid = min(KT, a.T - j0);
      tree_t = t - r.np;
    }
  };
  // Producer wave p (wave NW + p) copies plane p (0: K, 1: V) of every tile,
  // NINSTR 1 KB copies per tile.  Rows past the valid ones of a partial tile
  // repeat its last valid row; they are masked.
  const int pw = wave - NW;
  auto issue_tile = [&](const Cur& r, int64_t x, int st) {
    const uint16_t *kb, *vb;
    int nvalid, tree_t;
    tile_src(r, x, kb, vb, nvalid, tree_t);
    const uint16_t* src = pw == 0 ? kb : vb;
    unsigned char* dst = lds + st * TL::STAGEB + (pw == 0 ? 0 : TL::TILEB);
#pragma unroll
    for (int ins = 0; ins < TL::NINSTR; ++ins) {
      const int row = ins * TL::RPI + lane / TL::CPR;
      const int slot = lane % TL::CPR;
      const int sw = pw == 0 ? TL::swz_k(row) : TL::swz_v(row);
      const int srow = nvalid == KT ? row : min(row, nvalid - 1);
      copy16_to_lds(src + srow * D + 8 * (slot ^ sw), dst + ins * 1024);
    }
  };

  int koff[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) koff[ks] = n16 * TL::ROWB + 16 * ((ks * 4 + grp) ^ TL::swz_k(n16));
  const int vrow = 4 * grp + (n16 >> 2);
  const int q4 = lane & 3;
  int voff[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
    voff[dt] = vrow * TL::ROWB + 16 * ((2 * dt + (q4 >> 1)) ^ TL::swz_v(vrow)) + 8 * (q4 & 1);
  // With eight compute waves (two per SIMD, bound by the SIMDs' issue) the
  // tile loop is unrolled over the four ring stages, so that each stage's LDS
  // offsets sit in the read instructions; stages 2 and 3 lie beyond their
  // 16-bit offset field and read from these copies of the lane offsets moved
  // up by two stages (B=1 32K: 24 fewer VALU instructions per tile, 1-3 %
  // faster, bitwise the same; with nine waves, whose registers are short, 2 %
  // slower, and with two, bound by memory, no faster).
  constexpr bool kStaticStages = NW * QMAX == 8;
  int koff_hi[kStaticStages ? NKS : 1], voff_hi[kStaticStages ? NDT : 1];
  if constexpr (kStaticStages) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      koff_hi[ks] = koff[ks] + 2 * TL::STAGEB;
      asm volatile("" : "+v"(koff_hi[ks]));  // kept in registers, not folded back
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      voff_hi[dt] = voff[dt] + 2 * TL::STAGEB;
      asm volatile("" : "+v"(voff_hi[dt]));
    }
  }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
  const float sc = a.scale_log2;

  // Per-piece state of this wave's query tiles (block tiles wave, wave + NW, ...).
  bf16x8 qf[QMAX][NKS];
  f32x4 o[QMAX][NDT];
  f32x4 lacc[QMAX];
  float m_ref[QMAX];
  int row_node[QMAX], row_head[QMAX];

  Cur cur{}, pcur{};
  if (lo < hi) {
    cur = locate(lo);
    pcur = cur;
  }
  if (small_b) __syncthreads();  // wave 0's LDS table, read from here on
  if (c == 0 && a.ws_pref)
    for (int b = tid; b <= B; b += NT) {
      a.ws_pref[b] = s_pref[b];
      a.ws_pref[B + 1 + b] = s_npref[b];
    }
  // Producer cursor: pcur/px walk the range ahead of the compute waves.
  int64_t px = lo;
  auto produce = [&](int st) {
    if (px == pcur.base + pcur.ntl) advance(pcur);
    issue_tile(pcur, px, st);
    ++px;
  };
  // Tile y is visible to the compute waves after barrier y (one barrier per
  // tile for every wave of the workgroup; the producers pass it once their
  // copies of tile y are done).
  auto landed = [&](int64_t) { lds_barrier(); };

  // Scores of stream tile y for NQ query tiles: s[qt][u][e] = score of key
  // 16u + 4*grp + e of the tile for query n16.
  auto scores = [&](auto nq_c, int st, f32x4 (&sacc)[decltype(nq_c)::value][4]) {
    constexpr int NQ = decltype(nq_c)::value;
    const unsigned char* kl = lds + (kStaticStages ? st & 1 : st) * TL::STAGEB;
    const int* koffs = kStaticStages && st >= 2 ? koff_hi : koff;
#pragma unroll
    for (int qt = 0; qt < NQ; ++qt)
#pragma unroll
      for (int u = 0; u < 4; ++u) sacc[qt][u] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (NW * QMAX <= 9) {
      // K fragments eight at a time: their LDS reads are in flight together
      // before the first of their MFMAs waits, instead of one read and one
      // wait per MFMA (the 12-wave form has no registers to spare for this)
#pragma unroll
      for (int kb = 0; kb < NKS; kb += 2) {
        bf16x8 kf[2][4];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int u = 0; u < 4; ++u)
            kf[k2][u] = *reinterpret_cast<const bf16x8*>(kl + 16 * u * TL::ROWB + koffs[kb + k2]);
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int qt = 0; qt < NQ; ++qt)
#pragma unroll
            for (int u = 0; u < 4; ++u)
              sacc[qt][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[k2][u], qf[qt][kb + k2], sacc[qt][u], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int qt = 0; qt < NQ; ++qt)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int u = 0; u < 4; ++u)
            sacc[qt][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                *reinterpret_cast<const bf16x8*>(kl + 16 * u * TL::ROWB + koffs[ks]), qf[qt][ks], sacc[qt][u], 0, 0, 0);
    }
  };
  // Mask, softmax and P V of stream tile y from its scores.
  auto finish = [&](auto nq_c, int st, int64_t y, f32x4 (&sacc)[decltype(nq_c)::value][4]) {
    constexpr int NQ = decltype(nq_c)::value;
    const uint16_t *kb_, *vb_;
    int nvalid, tree_t;
    tile_src(cur, y, kb_, vb_, nvalid, tree_t);
    const unsigned char* vl = lds + (kStaticStages ? st & 1 : st) * TL::STAGEB + TL::TILEB;
    const int* voffs = kStaticStages && st >= 2 ? voff_hi : voff;
    if (tree_t >= 0 || nvalid < KT) {  // wave-uniform, rare
      const uint64_t head_bits = nvalid >= 64 ? ~0ull : ((1ull << nvalid) - 1ull);
#pragma unroll
      for (int qt = 0; qt < NQ; ++qt) {
        uint64_t v = row_node[qt] >= 0 ? head_bits : 0ull;
        if (tree_t >= 0) v &= s_mask[(wave + NW * qt) * 16 + n16][tree_t];
        const uint64_t bits = v >> (4 * grp);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (!((bits >> (16 * u + e)) & 1ull)) sacc[qt][u][e] = kNegInf;
      }
    }
    float mx[NQ];
    bool up = false;
#pragma unroll
    for (int qt = 0; qt < NQ; ++qt) {
      float m = sacc[qt][0][0];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = fmaxf(m, sacc[qt][u][e]);
      mx[qt] = m * sc;
      up = up || (mx[qt] > m_ref[qt] + kRescale);
    }
    if (__any(up)) {  // one wave-uniform branch per key tile; first tiles, then rare
#pragma unroll
      for (int qt = 0; qt < NQ; ++qt) {
        const float m_new = fmaxf(m_ref[qt], group_max(mx[qt]));
        if (m_new > m_ref[qt] + kRescale || m_ref[qt] == kNegInf) {
          const float alpha = m_new == kNegInf ? 1.0f : __builtin_amdgcn_exp2f(m_ref[qt] - m_new);
          lacc[qt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[qt][dt] *= alpha;
          m_ref[qt] = m_new;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const unsigned char* vh = vl + 32 * h * TL::ROWB;
      bf16x8 vf[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vh + voffs[dt]));
        const s16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vh + 16 * TL::ROWB + voffs[dt]));
        vf[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int qt = 0; qt < NQ; ++qt) {
        const float neg_m = m_ref[qt] == kNegInf ? 0.0f : -m_ref[qt];
        bf16x8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pf[e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[qt][2 * h + e / 4][e % 4], sc, neg_m));
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          o[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pf, o[qt][dt], 0, 0, 0);
        lacc[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf, lacc[qt], 0, 0, 0);
      }
    }
  };

  // The tiles of one piece for a compute wave with NQ live query tiles.  A
  // wave is done with tile x before it arrives at barrier x + 1, which lets
  // the producers refill that stage right after the barrier (three tiles in
  // flight with four stages); the matrix cores overlap the softmax of one
  // wave with the MFMAs of the others.  Each piece runs one instance, so the
  // accumulators keep their registers.
  auto run_piece = [&](auto nq_c, int64_t x0, int64_t x1) {
    constexpr int NQ = decltype(nq_c)::value;
    if constexpr (NQ == 0) {
      for (int64_t x = x0; x < x1; ++x) landed(x);
    } else {
      f32x4 sa[NQ][4];
      if (!lag) {
        auto step = [&](int st, int64_t x) __attribute__((always_inline)) {
          landed(x);
          scores(nq_c, st, sa);
          finish(nq_c, st, x, sa);
        };
        int64_t x = x0;
        if constexpr (kStaticStages) {
          for (; x < x1 && (x - lo) % kStages != 0; ++x) step((int)((x - lo) % kStages), x);
          for (; x + kStages <= x1; x += kStages) {
            static_assert(kStages == 4, "the unrolled loop names four stages");
            step(0, x);
            step(1, x + 1);
            step(2, x + 2);
            step(3, x + 3);
          }
        }
        for (; x < x1; ++x) step((int)((x - lo) % kStages), x);
      } else {
        // Lagging wave: between barriers x and x + 1 it finishes tile x - 1
        // (softmax, P V) and then computes the scores of tile x, so its
        // matrix work falls where the leading waves run their softmax.
        for (int64_t x = x0; x < x1; ++x) {
          landed(x);
          if (x > x0) finish(nq_c, (int)((x - 1 - lo) % kStages), x - 1, sa);
          scores(nq_c, (int)((x - lo) % kStages), sa);
        }
        finish(nq_c, (int)((x1 - 1 - lo) % kStages), x1 - 1, sa);
      }
    }
  };


  if (wave >= NW) {
    // Producer of K: three tiles ahead.  Before barrier y it waits for its
    // copies of tile y (tiles y + 1 and y + 2 may still be in flight); after
    // it, it issues tile y + 3 into the stage of tile y - 1, whose K every
    // compute wave read before arriving at barrier y.  Producer of V: two
    // tiles ahead when some compute waves lag (they read V of tile y - 1
    // between barriers y and y + 1), so tile y + 2 goes into the stage of
    // tile y - 2; three ahead otherwise.
    const bool two_ahead = pw == 1 && kLagging;
    if (lo < hi) produce(0);
    if (lo + 1 < hi) produce(1);
    if (!two_ahead && lo + 2 < hi) produce(2);
    for (int64_t y = lo; y < hi; ++y) {
      if (!two_ahead && y + 2 < hi) wait_vmcnt<2 * TL::NINSTR>();
      else if (y + 1 < hi) wait_vmcnt<TL::NINSTR>();
      else wait_vmcnt<0>();
      lds_barrier();
      if (two_ahead) {
        if (y + 2 < hi) produce((int)((y - lo + 2) % kStages));
      } else if (y + 3 < hi) {
        produce((int)((y - lo + 3) % kStages));
      }
    }
  } else
  for (int64_t x = lo; x < hi;) {
    // ---- a piece of unit `cur`: [x, pend)
    const int64_t pend = min(hi, cur.base + (int64_t)cur.ntl);
    const bool whole = x == cur.base && pend == cur.base + cur.ntl;
    const int g = cur.j / a.nqb, qb = cur.j % a.nqb;
    const int t0 = unit_tile_lo(a, qb);
    const int ntq = unit_tile_lo(a, qb + 1) - t0;  // query tiles of this unit
    const int r0 = 16 * t0;
    int nlive = 0;
#pragma unroll
    for (int qt = 0; qt < QMAX; ++qt) {
      const int lt = wave + NW * qt;
      const bool live = lt < ntq;
      nlive += live ? 1 : 0;
      const int r = r0 + lt * 16 + n16;
      const bool ok = live && r < a.R;
      row_node[qt] = ok ? r % a.T : -1;
      row_head[qt] = ok ? g * a.G + r / a.T : 0;
      const uint16_t* qrow = q + (((int64_t)cur.b * a.T + (ok ? row_node[qt] : 0)) * a.Hq + row_head[qt]) * D;
      // the row's mask words and its Q fragments are loaded together and
      // waited for once
      const uint64_t* mr = a.mask + ((int64_t)cur.b * a.T + (ok ? row_node[qt] : 0)) * a.W;
      uint64_t mw[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) mw[w] = (ok && w < a.W) ? mr[w] : 0ull;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if (ok) {
          qf[qt][ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 32 + grp * 8);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) qf[qt][ks][e] = (__bf16)0.0f;
        }
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) settle(qf[qt][ks]);
      if (live)
#pragma unroll
        for (int w = 0; w < 4; ++w)
          if (w < a.W) s_mask[lt * 16 + n16][w] = mw[w];
      m_ref[qt] = row_node[qt] >= 0 ? kNegInf : 0.0f;
      lacc[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    nlive = __builtin_amdgcn_readfirstlane(nlive);
    if (x == cur.base && cur.j == 0 && tid == 0 && a.seq_status) a.seq_status[cur.b] = SVT_OK;

    if (QMAX >= 2 && nlive == 2) run_piece(std::integral_constant<int, (QMAX >= 2 ? 2 : 1)>{}, x, pend);
    else if (nlive == 1) run_piece(std::integral_constant<int, 1>{}, x, pend);
    else run_piece(std::integral_constant<int, 0>{}, x, pend);

    // ---- end of the piece; lane holds O^T[d = dt*16 + 4*grp + e][query n16]
    // A cut piece leaves its normalised output O / l in fp16, divided by the
    // row's largest |O / l| (s, kept in fp32 with m and l): the stored values
    // lie in [-1, 1], so their rounding error is at most 2^-12 s, an eighth of
    // the bf16 output's relative rounding, whatever the scale of V.
    float pscale[QMAX];
#pragma unroll
    for (int qt = 0; qt < QMAX; ++qt) {
      float am = 0.0f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) am = fmaxf(am, fabsf(o[qt][dt][e]));
      pscale[qt] = whole ? 0.0f : group_max(am);  // all lanes: the four lanes of a row exchange
    }
#pragma unroll
    for (int qt = 0; qt < QMAX; ++qt) {
      if (qt >= nlive) continue;
      const bool rowok = row_node[qt] >= 0;  // rows past R: no output, no partial
      const int lt = wave + NW * qt;
      if (whole) {
        if (!rowok) continue;
        const float inv = 1.0f / lacc[qt][0];
        __bf16* orow = static_cast<__bf16*>(a.out) + (((int64_t)cur.b * a.T + row_node[qt]) * a.Hq + row_head[qt]) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[qt][dt][e] * inv);
          *reinterpret_cast<bf16x4*>(orow + dt * 16 + 4 * grp) = v;
        }
      } else {
        const int slot = 2 * c + ((pend == hi && pend < cur.base + cur.ntl) ? 1 : 0);
        const int64_t pr = (int64_t)slot * a.qb_rows + lt * 16 + n16;
        const float l = lacc[qt][0];
        const float s_row = l > 0.0f ? pscale[qt] / l : 0.0f;      // max |O / l| of the row
        const float f = pscale[qt] > 0.0f ? 1.0f / pscale[qt] : 0.0f;  // O -> (O / l) / s
        typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
        _Float16* po = a.ws_h + pr * D;
        f16x4 v16[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int e = 0; e < 4; ++e) v16[dt][e] = (_Float16)(o[qt][dt][e] * f);
        const float4 mls = make_float4(m_ref[qt], l, s_row, 0.0f);
        if (rowok) {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f16x4*>(po + dt * 16 + 4 * grp) = v16[dt];
          if (grp == 0) a.ws_mls[pr] = mls;
        }
      }
    }
    x = pend;
    if (x < hi) advance(cur);
  }

  // ---- skipped sequences: zero output rows and report why (ranges share the work)
  for (int b = c; b < B; b += NG) {
    if (s_pref[b + 1] != s_pref[b]) continue;
    int code;
    stream_seq_tiles(a, b, lmax, &code);
    __bf16* out = static_cast<__bf16*>(a.out) + (int64_t)b * a.T * a.Hq * D;
    for (int i = tid; i < a.T * a.Hq * D; i += NT) out[i] = (__bf16)0.0f;
    if (tid == 0 && a.seq_status) a.seq_status[b] = code;
  }
}

// Merges the partials of the units that range ends cut, in stream order.
// Grid (range, group of rows): D / DPT threads per row, DPT dims each (the
// launch picks DPT so that the grid covers the chip).  A cut unit is merged by
// the workgroups of the first range holding its tiles.  That range's record
// (written by the main kernel) names the unit and its last range; it is loaded together with the partials of the two
// pieces of a unit cut once (slots 2c + 1 and 2c + 2), so such a unit costs
// one memory round trip.  A
// unit spread over more ranges lists the rest of its pieces (empty ranges
// skipped) in LDS, one range per lane, and merges them in batches of
// KB = 32 / DPT pieces (4 at 16 dims).  With a whole number of ranges per unit (one
// sequence) the pieces are known without the record: see below.
constexpr int kMaxPieces = 64;  // pieces listed per pass (one wave)

template <int D, int DPT>
__global__ __launch_bounds__(256) void attn_stream_combine_kernel(AttnDev a) {
  constexpr int TPR = D / DPT;   // threads per row
  constexpr int RPW = 256 / TPR; // rows per workgroup
  constexpr int KB = DPT >= 16 ? 4 : 32 / DPT;  // pieces loaded per batch
  typedef _Float16 f16xN __attribute__((ext_vector_type(DPT)));
  int cr = blockIdx.x;  // range (with a whole number of ranges per unit: the unit)
  const int G = a.stream_grid;
  const int rl = blockIdx.y * RPW + threadIdx.x / TPR;
  const int d0 = (threadIdx.x % TPR) * DPT;
  const int rld = min(rl, a.qb_rows - 1);  // row the loads use (in the slot whatever rl is)
  // Row rld of partial slot `slot`: (m, l, s) and DPT dims of O / (l s).
  auto load_piece = [&](int64_t slot, float& mi, float& li, float& si, float (&oi)[DPT]) {
    const int64_t pr = slot * a.qb_rows + rld;
    const float4 mls = a.ws_mls[pr];
    mi = mls.x;
    li = mls.y;
    si = mls.z;
    const f16xN v = *reinterpret_cast<const f16xN*>(a.ws_h + pr * D + d0);
#pragma unroll
    for (int e = 0; e < DPT; ++e) oi[e] = (float)v[e];
  };
  // The unit's output row r of query block qb, or false for rows past it.
  auto unit_row = [&](int u, int& b, int& g, int& r) {
    const int qb = u % a.nqb, bg = u / a.nqb;
    g = bg % a.Hkv;
    b = bg / a.Hkv;
    const int t0 = unit_tile_lo(a, qb);
    r = 16 * t0 + rl;
    return rl < 16 * (unit_tile_lo(a, qb + 1) - t0) && r < a.R;
  };
  auto store_row = [&](int b, int g, int r, const float (&acc)[DPT], float l) {
    const float inv = 1.0f / l;
    __bf16* orow = static_cast<__bf16*>(a.out) + (((int64_t)b * a.T + r % a.T) * a.Hq + g * a.G + r / a.T) * D;
    if constexpr (DPT % 4 == 0) {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int e = 0; e < DPT; e += 4) {
        bf16x4 v;
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = (__bf16)(acc[e + k] * inv);
        *reinterpret_cast<bf16x4*>(orow + d0 + e) = v;
      }
    } else {
#pragma unroll
      for (int e = 0; e < DPT; ++e) orow[d0 + e] = (__bf16)(acc[e] * inv);
    }
  };

  if (a.rpu > 0) {
    // One sequence, a whole number of ranges per unit: when every range
    // holds tiles of the unit, unit u's pieces are those of ranges u * rpu ..
    // u * rpu + rpu - 1 (slot 2c + 1, the last one 2c), so the unit's
    // workgroups merge them with no record and no list, the
    // first batch of partials requested together with the sequence's tile
    // count (its slots exist in any case).  The grid then has one workgroup
    // per unit and group of rows.
    const int np = a.rpu;
    const int u = cr;
    float mi[KB], li[KB], si[KB];
    float oi[KB][DPT];
    auto load_batch = [&](int k) {
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const int kk = min(k + j, np - 1);
        load_piece(2 * ((int64_t)u * np + kk) + (kk < np - 1 ? 1 : 0), mi[j], li[j], si[j], oi[j]);
      }
    };
    load_batch(0);
    const int ntl1 = a.ws_pref[1] - a.ws_pref[0];
    if (ntl1 == 0) return;  // the sequence was skipped: no partials, zeros are written
    const int PC1 = a.piece_cost;
    if ((ntl1 + PC1) / np >= PC1 + 2) {  // every range holds at least one tile of the unit
      int b, g, r;
      if (!unit_row(u, b, g, r)) return;
      float mx = kNegInf, l = 0.0f;
      float acc[DPT];
#pragma unroll
      for (int e = 0; e < DPT; ++e) acc[e] = 0.0f;
      for (int k = 0; k < np; k += KB) {
        if (k > 0) load_batch(k);
#pragma unroll
        for (int j = 0; j < KB; ++j) {
          if (k + j >= np) break;
          merge_piece(mx, l, acc, mi[j], li[j], si[j], oi[j]);
        }
      }
      store_row(b, g, r, acc, l);
      return;
    }
    // Some ranges of the unit hold no tile (a short sequence): its pieces
    // are found from the record of its first cut range, among its own ranges.
    int c0 = -1;
    for (int c = u * np; c < (u + 1) * np; ++c)
      if (a.ws_meta[c].u == u) {
        c0 = c;
        break;
      }
    if (c0 < 0) return;  // the unit lies in one range: written directly
    cr = c0;
  }

  // ---- the record of range cr, and the partials a unit cut once uses
  const RangeMeta m = a.ws_meta[cr];
  float m0, l0, s0, o0[DPT], m1, l1, s1, o1[DPT];
  load_piece(2 * (int64_t)cr + 1, m0, l0, s0, o0);
  load_piece(min(2 * (int64_t)cr + 2, 2 * (int64_t)G - 1), m1, l1, s1, o1);
  if (m.u < 0) return;  // workgroup-uniform
  int b, g, r;
  const bool row_ok = unit_row(m.u, b, g, r);
  // Online merge in range order (deterministic): this range's piece first.
  float mx = kNegInf, l = 0.0f;
  float acc[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) acc[e] = 0.0f;
  merge_piece(mx, l, acc, m0, l0, s0, o0);
  if (m.c1 == cr + 1) {
    if (!row_ok) return;
    merge_piece(mx, l, acc, m1, l1, s1, o1);
    store_row(b, g, r, acc, l);
    return;
  }
  // ---- a unit over three or more ranges: list the pieces of ranges
  // cr + 1 .. c1 (ranges between may be empty when there are fewer tiles than
  // ranges) and merge them in batches
  const UnitCut uc = unit_cut(m.ct, m.cu, m.p, G, a.piece_cost, m.ntl);
  __shared__ int s_slot[kMaxPieces];
  __shared__ int s_np;
  for (int cs = cr + 1; cs <= m.c1; cs += kMaxPieces) {
    __syncthreads();
    if (threadIdx.x < kMaxPieces) {
      const int cc = cs + (int)threadIdx.x;
      int slot = 0;
      const bool has = cc <= m.c1 && unit_piece(uc, cc, &slot);
      const uint64_t bal = __ballot(has);
      const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      if (has) s_slot[below] = slot;
      if (threadIdx.x == 0) s_np = (int)__popcll(bal);
    }
    __syncthreads();
    if (!row_ok) continue;
    const int np = s_np;
    for (int k = 0; k < np; k += KB) {
      float mi[KB], li[KB], si[KB];
      float oi[KB][DPT];  // converted on load: the merge loop below indexes it
      // every slot loads (past the last piece: the last piece again), so the
      // batch's loads issue back to back; only the real pieces are merged
#pragma unroll
      for (int j = 0; j < KB; ++j) load_piece(s_slot[min(k + j, np - 1)], mi[j], li[j], si[j], oi[j]);
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        if (k + j >= np) break;
        merge_piece(mx, l, acc, mi[j], li[j], si[j], oi[j]);
      }
    }
  }
  if (!row_ok) return;
  store_row(b, g, r, acc, l);
}

// --------------------------------------------------------------------------
// fp32 VALU kernel: one query row per wave, four per workgroup.
// --------------------------------------------------------------------------
// A row is a chain of dependent LDS reads (q . k, then P V, per key tile), so
// one row per wave and more workgroups keep the call short: B=1 fp32 (36
// rows, 137 keys) 21.6 -> 8.6 us against four rows per wave.
constexpr int kFp32RowsPerWave = 1;

template <int D>
__global__ __launch_bounds__(256) void attn_fp32_kernel(AttnDev a) {
  constexpr int DPL = D / 64;  // dims per lane
  constexpr int KS = D + 1;    // padded K row (floats) against bank conflicts
  constexpr int RPW = kFp32RowsPerWave;  // query rows per wave, handled one after another
  __shared__ __attribute__((aligned(16))) float qs[4 * RPW * D];
  __shared__ float ks[KT * KS];
  __shared__ float vs[KT * D];
  __shared__ __attribute__((aligned(16))) float ps[4][KT];
  __shared__ uint64_t mws[4 * RPW][4];

  WgCtx c;
  if (!decode_coords(a, c) || !decode_lengths(a, c)) return;
  write_seq_status(a, c);
  if (c.code != SVT_OK) {
    if (c.split == 0) write_zero_rows<float>(a, c, D);
    return;
  }
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float* __restrict__ q = static_cast<const float*>(a.q);
  const float* __restrict__ kc = static_cast<const float*>(a.kcache);
  const float* __restrict__ vc = static_cast<const float*>(a.vcache);
  const float* __restrict__ ktr = static_cast<const float*>(a.ktree);
  const float* __restrict__ vtr = static_cast<const float*>(a.vtree);
  const int64_t bg = (int64_t)c.b * a.Hkv + c.g;
  const int r0 = c.qb * 4 * RPW;

  const int n_tiles = c.n_ptiles + c.n_ttiles;
  const int pad = c.lmax - c.L;
  // Source rows of tile t: prefix columns, or (after the prefix) tree rows.
  auto tile_src = [&](int t, const float*& kb, const float*& vb, int& nvalid) {
    if (t < c.n_ptiles) {
      const int k0 = c.k_beg + t * KT;
      kb = kc + (c.cg * a.cap + pad + k0) * D;
      vb = vc + (c.cg * a.cap + pad + k0) * D;
      nvalid = min(KT, c.k_end - k0);
    } else {
      const int j0 = (t - c.n_ptiles) * KT;
      kb = ktr + (bg * a.T + j0) * D;
      vb = vtr + (bg * a.T + j0) * D;
      nvalid = min(KT, a.T - j0);
    }
  };
  // Tile t's K and V go to registers first (one 16-byte load per float4,
  // all in flight together); the next tile's loads are issued before the
  // current tile is computed on, so they overlap it.
  constexpr int PER = KT * D / 4 / 256;  // float4 of K (and of V) per thread
  float4 kr[PER], vr[PER];
  auto load_tile = [&](int t) {
    const float *kb, *vb;
    int nvalid;
    tile_src(t, kb, vb, nvalid);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int x = 4 * (tid + 256 * j), row = x / D, d = x % D;
      const bool ok = row < nvalid;  // rows past the valid ones are never read (they may not exist)
      kr[j] = ok ? *reinterpret_cast<const float4*>(kb + (int64_t)row * D + d) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      vr[j] = ok ? *reinterpret_cast<const float4*>(vb + (int64_t)row * D + d) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
  };
  if (n_tiles > 0) load_tile(0);
  // Global loads are issued together (16-byte loads, all in flight before
  // the first LDS write): one memory round trip per stage, not one per
  // element.  Rows are D floats, so every 4-float group lies in one row.
  {
    // ancestor-mask words of the block's rows, for the tree tiles (written
    // to LDS below, visible after the first tile's barrier)
    uint64_t mv = 0ull;
    if (c.n_ttiles > 0 && tid < 4 * RPW * 4) {
      const int rr = tid / 4, w = tid % 4, r = r0 + rr;
      if (r < a.R && w < a.W) mv = a.mask[((int64_t)c.b * a.T + r % a.T) * a.W + w];
    }
    constexpr int NQF4 = RPW * D;                // float4 of the block's Q rows (4 * RPW rows)
    constexpr int NQ4 = (NQF4 + 255) / 256;      // per thread
    float4 qr[NQ4];
#pragma unroll
    for (int j = 0; j < NQ4; ++j) {
      const int x = 4 * (tid + 256 * j), rr = x / D, d = x % D, r = r0 + rr;
      qr[j] = (tid + 256 * j < NQF4 && r < a.R)
                  ? *reinterpret_cast<const float4*>(q + (((int64_t)c.b * a.T + r % a.T) * a.Hq + c.g * a.G + r / a.T) * D + d)
                  : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int j = 0; j < NQ4; ++j)
      if (tid + 256 * j < NQF4) *reinterpret_cast<float4*>(qs + 4 * (tid + 256 * j)) = qr[j];
    if (c.n_ttiles > 0 && tid < 4 * RPW * 4) mws[tid / 4][tid % 4] = mv;
  }
  float m_run[RPW], l_run[RPW], o[RPW][DPL];
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    m_run[j] = kNegInf;
    l_run[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[j][e] = 0.0f;
  }
  for (int t = 0; t < n_tiles; ++t) {
    const float *kb_, *vb_;
    int nvalid;
    tile_src(t, kb_, vb_, nvalid);
    const bool tree_tile = t >= c.n_ptiles;
    __syncthreads();  // the previous tile's readers are done
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int x = 4 * (tid + 256 * j), row = x / D, d = x % D;
      float* kd = ks + row * KS + d;
      kd[0] = kr[j].x;
      kd[1] = kr[j].y;
      kd[2] = kr[j].z;
      kd[3] = kr[j].w;
      *reinterpret_cast<float4*>(vs + x) = vr[j];
    }
    __syncthreads();
    if (t + 1 < n_tiles) load_tile(t + 1);
#pragma unroll 1
    for (int j = 0; j < RPW; ++j) {
      const int rr = wave * RPW + j, r = r0 + rr;
      if (r >= a.R) break;  // wave-uniform
      const int node = r % a.T;
      bool ok = lane < nvalid;
      if (tree_tile) {
        const uint64_t mw = mws[rr][t - c.n_ptiles];
        ok = ok && ((mw >> lane) & 1ull);
      }
      // q . k in four interleaved partial sums (a quarter of the dependent
      // chain); the Q row is read four floats at a time (an LDS broadcast)
      const float* qp = qs + rr * D;
      const float* kp = ks + lane * KS;
      float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int d = 0; d < D; d += 4) {
        const float4 qv = *reinterpret_cast<const float4*>(qp + d);
        s4[0] = fmaf(qv.x, kp[d], s4[0]);
        s4[1] = fmaf(qv.y, kp[d + 1], s4[1]);
        s4[2] = fmaf(qv.z, kp[d + 2], s4[2]);
        s4[3] = fmaf(qv.w, kp[d + 3], s4[3]);
      }
      const float s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
      const float x = ok ? s * a.scale_log2 : kNegInf;
      float tmax = x;
      for (int off = 32; off > 0; off >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off));
      const float m_new = fmaxf(m_run[j], tmax);
      const float m_use = m_new == kNegInf ? 0.0f : m_new;
      const float alpha = exp2f(m_run[j] - m_use);
      const float p = exp2f(x - m_use);
      float psum = p;
      for (int off = 32; off > 0; off >>= 1) psum += __shfl_xor(psum, off);
      l_run[j] = l_run[j] * alpha + psum;
      m_run[j] = m_new;
      ps[wave][lane] = p;
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const int d = lane + 64 * e;
        float a4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < KT; k += 4) {
          const float4 pv = *reinterpret_cast<const float4*>(&ps[wave][k]);
          a4[0] = fmaf(pv.x, vs[k * D + d], a4[0]);
          a4[1] = fmaf(pv.y, vs[(k + 1) * D + d], a4[1]);
          a4[2] = fmaf(pv.z, vs[(k + 2) * D + d], a4[2]);
          a4[3] = fmaf(pv.w, vs[(k + 3) * D + d], a4[3]);
        }
        o[j][e] = o[j][e] * alpha + ((a4[0] + a4[1]) + (a4[2] + a4[3]));
      }
    }
  }
  const bool direct = c.ns_b == 1;
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int r = r0 + wave * RPW + j;
    if (r >= a.R) break;
    if (direct) {
      float* orow = static_cast<float*>(a.out) + (((int64_t)c.b * a.T + r % a.T) * a.Hq + c.g * a.G + r / a.T) * D;
#pragma unroll
      for (int e = 0; e < DPL; ++e) orow[lane + 64 * e] = o[j][e] / l_run[j];
    } else {
      const int64_t pr = (bg * a.ns + c.split) * a.R + r;
#pragma unroll
      for (int e = 0; e < DPL; ++e) a.ws_o[pr * D + lane + 64 * e] = o[j][e];
      if (lane == 0) {
        a.ws_ml[pr * 2 + 0] = m_run[j];
        a.ws_ml[pr * 2 + 1] = l_run[j];
      }
    }
  }
}

// --------------------------------------------------------------------------
// Split combine: one wave per query row, splits merged in index order.
// --------------------------------------------------------------------------
template <int D, typename E, int KB>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnDev a) {
  constexpr int DPL = D / 64;
  const int b = blockIdx.z, g = blockIdx.y;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= a.R) return;
  const int64_t base = ((int64_t)b * a.Hkv + g) * a.ns;
  // The partials of the first KB splits are loaded together with the
  // sequence's lengths (their slots exist whatever the lengths are; slots of
  // splits the sequence does not use are loaded and ignored), so a call with
  // at most KB splits pays one memory round trip before the merge.  The
  // arithmetic runs in split order: the maximum, then the weighted sums
  // (fused multiply-adds, whatever the batch of loads).
  float mv[KB], lv[KB], ov[KB][DPL];
#pragma unroll
  for (int j = 0; j < KB; ++j) {
    const int64_t pr = (base + min(j, a.ns - 1)) * a.R + r;
    mv[j] = a.ws_ml[pr * 2];
    lv[j] = a.ws_ml[pr * 2 + 1];
#pragma unroll
    for (int e = 0; e < DPL; ++e) ov[j][e] = a.ws_o[pr * D + lane + 64 * e];
  }
  const int lmax = *a.lmax;
  const int L = a.len[b];
  if (seq_code(a, b, lmax, L) != SVT_OK) return;
  const int ns_b = max(1, (L + a.kc - 1) / a.kc);
  if (ns_b <= 1) return;
  const int n0 = min(ns_b, KB);
  float mx = kNegInf;
#pragma unroll
  for (int j = 0; j < KB; ++j)
    if (j < n0) mx = fmaxf(mx, mv[j]);
  for (int s0 = KB; s0 < ns_b; s0 += KB) {
    float mw[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) mw[j] = s0 + j < ns_b ? a.ws_ml[((base + s0 + j) * a.R + r) * 2] : kNegInf;
#pragma unroll
    for (int j = 0; j < KB; ++j) mx = fmaxf(mx, mw[j]);
  }
  const float mu = mx == kNegInf ? 0.0f : mx;
  float lsum = 0.0f, acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.0f;
#pragma unroll
  for (int j = 0; j < KB; ++j) {
    if (j >= n0) break;
    const float w = exp2f(mv[j] - mu);
    lsum = fmaf(lv[j], w, lsum);
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = fmaf(ov[j][e], w, acc[e]);
  }
  for (int s0 = KB; s0 < ns_b; s0 += KB) {
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int64_t pr = (base + min(s0 + j, ns_b - 1)) * a.R + r;
      mv[j] = a.ws_ml[pr * 2];
      lv[j] = a.ws_ml[pr * 2 + 1];
#pragma unroll
      for (int e = 0; e < DPL; ++e) ov[j][e] = a.ws_o[pr * D + lane + 64 * e];
    }
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      if (s0 + j >= ns_b) break;
      const float w = exp2f(mv[j] - mu);
      lsum = fmaf(lv[j], w, lsum);
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] = fmaf(ov[j][e], w, acc[e]);
    }
  }
  E* orow = static_cast<E*>(a.out) + (((int64_t)b * a.T + r % a.T) * a.Hq + g * a.G + r / a.T) * D;
  const float inv = 1.0f / lsum;
#pragma unroll
  for (int e = 0; e < DPL; ++e) orow[lane + 64 * e] = E(acc[e] * inv);
}

// --------------------------------------------------------------------------
// host side
// --------------------------------------------------------------------------
// Compute units of the current device (cached per device).
static int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cached[dev] = n;
  return n;
}

// Stream-form workspace: the prefix table, then the range records, then the
// partials' (m, l, s) and their fp16 rows.
static size_t stream_pref_bytes(int B) { return ((size_t)2 * (B + 1) * sizeof(int) + 255) / 256 * 256; }
static size_t stream_meta_bytes(int grid) { return ((size_t)grid * sizeof(RangeMeta) + 255) / 256 * 256; }

bool plan_attention(const svt_attn_args* a, AttnPlan* p) {
  if (!a || a->B < 0 || a->M < 0 || a->M >= SVT_MAX_T || a->Hq <= 0 || a->Hkv <= 0 || a->Hq % a->Hkv != 0 ||
      (a->D != 64 && a->D != 128) || (a->dtype != SVT_FP32 && a->dtype != SVT_BF16) || a->cap < 0 ||
      a->form < SVT_ATTN_AUTO || a->form > SVT_ATTN_STREAM ||
      a->lmax_bound < 0 || (int64_t)a->lmax_bound > a->cap || a->split_keys < 0 || a->split_keys % KT != 0 ||
      (a->split_keys > 0 && a->form == SVT_ATTN_STREAM))
    return false;
  p->T = a->M + 1;
  p->G = a->Hq / a->Hkv;
  p->R = p->G * p->T;
  p->nqt = (p->R + 15) / 16;
  p->grid = 0;
  p->rpu = 0;
  p->piece_cost = 0;
  // Key tiles the stream form would hold at most (host bound).
  const int64_t stream_tiles = (int64_t)a->B * a->Hkv * ((p->nqt + 11) / 12) *
                               (((int64_t)a->lmax_bound + KT - 1) / KT + (p->T + KT - 1) / KT);
  const int cus = a->dtype == SVT_BF16 ? device_cu_count() : 0;
  const bool stream_ok = a->B <= kStreamMaxB;
  // The stream form from two D=128 key tiles' worth of bytes per CU on (GQA
  // 32/8, D=128, M=32, equal lengths, split against stream: at one tile per CU
  // the split form is faster by up to 30 %, at two they are within 10 % of
  // each other, from four on the stream form is 15-40 % faster, e.g. B=16 of
  // 512 keys 35.2 -> 20.7 us and B=1 of 8192 keys 34.8 -> 25.1 us; at D=64,
  // whose tiles hold half the bytes, B=4 of up to 2048 keys, about two tiles
  // per CU: split 15.4 us, stream 19.1 us).
  bool use_stream = stream_ok && stream_tiles * a->D >= 2 * 128 * (int64_t)cus;
  // At most 64 query rows per KV head (MHA, say), so that the split form too
  // reads each key once, and at least four (sequence, KV head) pairs per CU:
  // the split form, which skips the stream form's per-unit set-up and merge
  // (MHA 32/32, M=16: B=128 of up to 256 keys 116.6 -> 105.0 us, at D=64
  // 81.0 -> 54.4 us; B=64 of up to 1024 keys 171.1 -> 163.0 us; MHA 16/16, M=32:
  // B=64 of up to 1024 keys 96.9 -> 90.2 us; within 2 % either way at B=32 of up
  // to 4096 keys, and 10-20 % slower below four pairs per CU).
  if (p->R <= 64 && (int64_t)a->B * a->Hkv >= 4 * (int64_t)cus) use_stream = false;
  if (a->form == SVT_ATTN_SPLIT || a->split_keys > 0) use_stream = false;
  if (a->form == SVT_ATTN_STREAM) {
    if (a->dtype != SVT_BF16 || !stream_ok) return false;
    use_stream = true;
  }
  if (a->dtype == SVT_BF16 && !use_stream) {
    // Very many sequences or a stream too short to give every CU two
    // tiles: the split form, four waves per workgroup; with one or two query
    // tiles two waves share the rows and split every key tile.
    p->wide = 0;
    p->nw = 4;
    p->qw = 1;
    p->nwk = p->nqt <= 2 ? 2 : 1;
    p->stages = 2;
    p->qb_rows = (p->nw / p->nwk) * p->qw * 16;
  } else if (a->dtype == SVT_BF16) {
    // Stream form: up to 12 query tiles per unit, spread evenly over the
    // fewest units per KV head, one tile per compute wave (plus the two
    // producer waves); one workgroup per CU.  With fewer units than CUs
    // units of at most 8 tiles are faster (B=1 32K 56.6 -> 53.8 us per call,
    // B=2 of up to 8192 keys 37.3 -> 27.7 us) as long as the K/V they read
    // twice stays in the 256 MB Infinity Cache; with more K/V the second
    // query block's reads go to HBM and 12 are faster (B=8 of up to 8192
    // keys 62.8 -> 52.2 us, B=16 106.1 -> 80.3 us, B=4 of up to 16384 keys
    // 64.9 -> 56.7 us).  The K/V bound is the host's: B Hkv lmax_bound rows
    // of K and V.
#ifndef SVT_STREAM_FEW_TPB
#define SVT_STREAM_FEW_TPB 8
#endif
    int cap_t = 12;
    const int64_t kv_bound = (int64_t)a->B * a->Hkv * a->lmax_bound * a->D * 4;
    if ((int64_t)a->B * a->Hkv * ((p->nqt + 11) / 12) < (int64_t)cus && kv_bound <= (int64_t)192 << 20)
      cap_t = SVT_STREAM_FEW_TPB;
    const int nqb = (p->nqt + cap_t - 1) / cap_t;
    const int tpb = (p->nqt + nqb - 1) / nqb;
    p->wide = 1;
    p->nw = tpb <= 2 ? tpb : tpb <= 4 ? 4 : tpb <= 6 ? 6 : tpb <= 8 ? 8 : tpb <= 9 ? 9 : 12;
    p->qw = 1;
    p->nqb = nqb;
    p->nwk = 1;
    p->stages = 4;
    p->qb_rows = tpb * 16;
    // A unit boundary inside a range costs the compute waves about five key
    // tiles' worth of time when nine or more of them store their pieces and
    // load the next piece's inputs at once, about two with fewer waves
    // (per-tile stamps for nine and more; call times over 0..4 for the one-
    // and two-tile forms); range cuts balance tiles plus this per unit.
    p->piece_cost = p->nw >= 9 ? 5 : 2;
    // One workgroup per CU.
    if (cus <= 0) return false;
    p->grid = cus;
    // With one sequence every unit holds the same tiles, so a grid of a whole
    // number of ranges per unit puts each range inside one unit and no range
    // pays a unit boundary (storing one piece, loading the next piece's Q);
    // it leaves fewer than `units` CUs idle, used only when that is at most
    // a tenth of them.
    const int units = a->Hkv * p->nqb;
    p->rpu = 0;
    if (a->B == 1 && units <= cus && 10 * units * (cus / units) >= 9 * cus) {
      p->grid = units * (cus / units);
      p->rpu = cus / units;
    }
  } else {
    p->wide = 0;
    p->nwk = 1;
    p->qw = 1;
    p->nw = 4;
    p->stages = 1;
    p->qb_rows = 4 * kFp32RowsPerWave;
  }
  if (!p->wide) p->nqb = (p->R + p->qb_rows - 1) / p->qb_rows;
  if (p->wide) {
    // Partials: two slots of qb_rows rows per range, plus the prefix of
    // tiles per sequence and one record per range.
    p->kc = 0;
    p->ns = 1;
    const size_t rows = (size_t)2 * p->grid * p->qb_rows;
    p->ws_bytes = stream_pref_bytes(a->B) + stream_meta_bytes(p->grid) + rows * (a->D * sizeof(_Float16) + sizeof(float4));
    return true;
  }
  // Prefix split size: enough workgroups to cover the chip several times over.
  const int64_t ptiles = ((int64_t)a->lmax_bound + KT - 1) / KT;
  const int64_t units = ptiles * a->B * a->Hkv * p->nqb;
  const int64_t target = 1024;
  int64_t tiles_per_split = (units + target - 1) / target;
  if (tiles_per_split < 4) tiles_per_split = 4;
  // a split size the caller fixes: the splits of a sequence no longer depend
  // on the batch
  if (a->split_keys > 0) tiles_per_split = a->split_keys / KT;
  p->kc = (int)(tiles_per_split * KT);
  p->ns = a->lmax_bound > 0 ? (int)((a->lmax_bound + p->kc - 1) / p->kc) : 1;
  if (p->ns < 1) p->ns = 1;
  p->ws_bytes = p->ns > 1 ? (size_t)a->B * a->Hkv * p->ns * p->R * (a->D + 2) * sizeof(float) : 0;
  return true;
}

hipError_t launch_attention(const svt_attn_args* a, const AttnPlan& p, hipStream_t s) {
  AttnDev d;
  d.q = a->q;
  d.kcache = a->k_cache;
  d.vcache = a->v_cache;
  d.ktree = a->k_tree;
  d.vtree = a->v_tree;
  d.mask = a->mask;
  d.len = a->len;
  d.lmax = a->lmax;
  d.status = a->status;
  d.slot = a->seq_slot;
  d.n_slots = a->seq_slot ? a->n_slots : a->B;
  d.out = a->out;
  d.seq_status = a->seq_status;
  if (p.wide) {
    unsigned char* w = static_cast<unsigned char*>(a->workspace);
    const size_t pref_bytes = stream_pref_bytes(a->B), meta_bytes = stream_meta_bytes(p.grid);
    const size_t rows = (size_t)2 * p.grid * p.qb_rows;
    d.ws_pref = reinterpret_cast<int*>(w);
    d.ws_meta = reinterpret_cast<RangeMeta*>(w + pref_bytes);
    d.ws_mls = reinterpret_cast<float4*>(w + pref_bytes + meta_bytes);
    d.ws_h = reinterpret_cast<_Float16*>(w + pref_bytes + meta_bytes + rows * sizeof(float4));
    d.ws_o = nullptr;
    d.ws_ml = nullptr;
  } else {
    float* ws = static_cast<float*>(a->workspace);
    const size_t n_o = p.ns > 1 ? (size_t)a->B * a->Hkv * p.ns * p.R * a->D : 0;
    d.ws_pref = nullptr;
    d.ws_meta = nullptr;
    d.ws_h = nullptr;
    d.ws_mls = nullptr;
    d.ws_o = ws;
    d.ws_ml = ws ? ws + n_o : nullptr;
  }
  d.stream_grid = p.grid;
  d.rpu = p.wide ? p.rpu : 0;
  d.piece_cost = p.piece_cost;
  d.cap = a->cap;
  d.B = a->B;
  d.T = p.T;
  d.Hq = a->Hq;
  d.Hkv = a->Hkv;
  d.G = p.G;
  d.R = p.R;
  d.W = (p.T + 63) / 64;
  d.lmax_bound = a->lmax_bound;
  d.kc = p.kc;
  d.ns = p.ns;
  d.nqb = p.nqb;
  d.qb_rows = p.qb_rows;
  d.nwk = p.nwk;
  d.nqt = p.nqt;
  const float scale = a->scale > 0.0f ? a->scale : 1.0f / sqrtf((float)a->D);
  d.scale_log2 = scale * kLog2e;
  if (p.wide) {
    // one workgroup per CU; with fewer ranges than CUs the rest get none,
    // and the XCD-aware range order keeps its multiple of 8
    const int cus = device_cu_count();
    const dim3 g(cus > p.grid ? cus : p.grid);
#define SVT_STREAM(DD)                                                                             \
  switch (p.nw) { /* compute waves; two producer waves on top */                                          \
    case 1: hipLaunchKernelGGL((attn_bf16_stream_kernel<DD, 1, 1>), g, dim3(3 * 64), 0, s, d); break;   \
    case 2: hipLaunchKernelGGL((attn_bf16_stream_kernel<DD, 2, 1>), g, dim3(4 * 64), 0, s, d); break;   \
    case 4: hipLaunchKernelGGL((attn_bf16_stream_kernel<DD, 4, 1>), g, dim3(6 * 64), 0, s, d); break;   \
    case 6: hipLaunchKernelGGL((attn_bf16_stream_kernel<DD, 6, 1>), g, dim3(8 * 64), 0, s, d); break;   \
    case 8: hipLaunchKernelGGL((attn_bf16_stream_kernel<DD, 8, 1>), g, dim3(10 * 64), 0, s, d); break;  \
    case 9: hipLaunchKernelGGL((attn_bf16_stream_kernel<DD, 9, 1>), g, dim3(11 * 64), 0, s, d); break;  \
    default: hipLaunchKernelGGL((attn_bf16_stream_kernel<DD, 12, 1>), g, dim3(14 * 64), 0, s, d); break; \
  }
    if (a->D == 128) { SVT_STREAM(128) } else { SVT_STREAM(64) }
#undef SVT_STREAM
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // One combine workgroup per (range, group of rows): the cut units are at
    // most one per range; with a whole number of ranges per unit, one per
    // (unit, group of rows).
    const int64_t nu = (int64_t)a->B * a->Hkv * p.nqb;
    if (nu > 0x7FFFFFF0) return hipErrorInvalidValue;
    const int64_t nwork = p.rpu > 0 ? nu : p.grid;
    // dims per thread: the largest of 16, 8, 4, 2 that still gives a working
    // workgroup per CU (B=1 32K: 4 dims, 7.4 -> 5.6 us per combine against 2,
    // which the rule asking two per CU gave; B=8 and B=32: 16 dims, 0.8 and
    // about 1 us per call less than 8; 32 dims were slower at both)
    const int want = p.grid;
    auto groups = [&](int k) { return nwork * ((p.qb_rows + 256 / (a->D / k) - 1) / (256 / (a->D / k))); };
    const int dpt = groups(16) >= want ? 16 : groups(8) >= want ? 8 : groups(4) >= want ? 4 : 2;
    const int rpw = 256 / (a->D / dpt);
    const dim3 cg((unsigned)(p.rpu > 0 ? nu : p.grid), (unsigned)((p.qb_rows + rpw - 1) / rpw));
#define SVT_COMBINE(DD)                                                                                   \
  if (dpt == 16) hipLaunchKernelGGL((attn_stream_combine_kernel<DD, 16>), cg, dim3(256), 0, s, d);        \
  else if (dpt == 8) hipLaunchKernelGGL((attn_stream_combine_kernel<DD, 8>), cg, dim3(256), 0, s, d);     \
  else if (dpt == 4) hipLaunchKernelGGL((attn_stream_combine_kernel<DD, 4>), cg, dim3(256), 0, s, d);     \
  else hipLaunchKernelGGL((attn_stream_combine_kernel<DD, 2>), cg, dim3(256), 0, s, d);
    if (a->D == 128) { SVT_COMBINE(128) } else { SVT_COMBINE(64) }
#undef SVT_COMBINE
    return hipGetLastError();
  }
  const int64_t nunits = (int64_t)a->B * a->Hkv * p.ns;
  if (nunits == 0) return hipSuccess;
  const int64_t nwg = 8 * p.nqb * ((nunits + 7) / 8);
  if (nwg > 0x7FFFFFF0) return hipErrorInvalidValue;
  d.nunits = (int)nunits;
  const unsigned grid = (unsigned)nwg;
  const dim3 block(256);
  if (a->dtype == SVT_BF16) {
#define SVT_ATTN_BF16(DD, QQ, SS, WW) \
  hipLaunchKernelGGL((attn_bf16_kernel<DD, QQ, SS, WW>), dim3(grid), dim3(WW * 64), 0, s, d)
#define SVT_ATTN_BF16_QW(DD, SS, WW) SVT_ATTN_BF16(DD, 1, SS, WW);
    if (a->D == 128) {
      SVT_ATTN_BF16_QW(128, 2, 4)
    } else {
      SVT_ATTN_BF16_QW(64, 2, 4)
    }
#undef SVT_ATTN_BF16_QW
#undef SVT_ATTN_BF16
  } else {
    if (a->D == 128) hipLaunchKernelGGL(attn_fp32_kernel<128>, dim3(grid), block, 0, s, d);
    else hipLaunchKernelGGL(attn_fp32_kernel<64>, dim3(grid), block, 0, s, d);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.ns <= 1) return e;
  const dim3 cgrid((p.R + 3) / 4, a->Hkv, a->B);
  // the first batch of splits, loaded in one round trip with the lengths,
  // covers every split when there are at most 16
#define SVT_COMBINE_S(DD, EE)                                                                          \
  if (p.ns <= 8) hipLaunchKernelGGL((attn_combine_kernel<DD, EE, 8>), cgrid, block, 0, s, d);         \
  else hipLaunchKernelGGL((attn_combine_kernel<DD, EE, 16>), cgrid, block, 0, s, d);
  if (a->dtype == SVT_BF16) {
    if (a->D == 128) { SVT_COMBINE_S(128, __bf16) } else { SVT_COMBINE_S(64, __bf16) }
  } else {
    if (a->D == 128) { SVT_COMBINE_S(128, float) } else { SVT_COMBINE_S(64, float) }
  }
#undef SVT_COMBINE_S
  return hipGetLastError();
}

}  // namespace svt
