// Chunked prefill (multi-query attention over the paged cache) for gfx950:
// the prefill kernel and the C ABI entry points that launch it.
//
// Sources: "PagedAttention por dentro" (blog.lo0.es), "Chunked prefill
// integrado con paged KV" (prefill chunks and decode share one step and one
// paged cache) and "Sliding window attention"; "Como funciona realmente
// vLLM" (alexanderzelada.com), "Que es el mecanismo de atencion"; "KV
// cache: la memoria de trabajo..." (blog.lo0.es), «Trucos para que el
// cuaderno sea más fino» (an 8-bit cache).
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>

#include "device_common.h"
#include "pagedkv.h"

namespace {

// ------------------------------------------------------------------ next: multi-query (chunked prefill), bf16
// Several new query tokens per sequence over the same paged cache: sequence
// b's chunk of n_b tokens holds the last n_b of its L_b cached positions
// (their K/V written before the call); chunk token i sits at position
// p = L_b - n_b + i and attends to positions 0..p (causal inside the chunk;
// with a sliding window of W tokens, p-W+1..p).  A decode step is the case
// n_b = 1.
//
// One workgroup of 8 wavefronts per (sequence, kv head, tile of query
// positions), two per SIMD.  The tile's score columns are (position,
// head-in-group) pairs, 256 of them (32 per wavefront, as two 16-column MFMA
// tiles), so 256 / g positions per tile.  The K and V tiles of SB consecutive
// blocks (one stage) are moved once per workgroup into LDS (three buffers:
// the stage being processed, the next one, whose scores are computed during
// this one, and the one after, being filled) and every wavefront reads them
// from there:
//   S^T = K . Q^T   v_mfma_f32_16x16x32_bf16, A = K piece j (16 tokens x 32
//                   channels, the cache's lane order), B = Q^T chunk j;
//   O  += P . V     v_mfma_f32_16x16x32_f16 over each pair of blocks (32
//                   tokens): a lane's k-index i < 4 is token 4(l/16)+i of the
//                   first block, i >= 4 the same token of the second block --
//                   the layout S^T comes out in, and the halves of the V
//                   tile's lane pieces of the two blocks;
// with P and V as f16 (V converted on its way into LDS; a bf16 V element
// beyond f16's range makes the workgroup run again with P as a bf16 high
// part plus residual and V as bf16).  The running max is raised only when a
// stage's max exceeds it by more than 2^8 (the normaliser uses the same
// reference, so the result is unchanged, and the accumulator is rescaled
// rarely).
struct PrefillArgs {
  const void* q;          // [T][Hq][D] bf16, T = qstart[B]
  const void* kc;
  const void* vc;
  const int32_t* tables;
  const int32_t* lens;
  const int32_t* qstart;  // [B + 1] first chunk row of each sequence
  float* out;             // [T][Hq][D] fp32
  int num_seqs, num_q_heads, num_kv_heads, group;
  int qtp;                // query positions per workgroup tile: 256 / group
  int tiles;              // tiles per sequence: ceil(max_query_len / qtp)
  int num_blocks, max_blocks, max_ctx;
  float scale_log2e;
  int window;  // sliding window in tokens: position p sees p-window+1 .. p (0: 0 .. p)
  float out_scale;  // 1, or the V scale of an FP8 cache
};

constexpr int kPfWaves = 8;
constexpr int kPfColTiles = 2;                       // 16-column tiles per wavefront
constexpr int kPfCols = kPfWaves * kPfColTiles * 16;  // score columns per workgroup
constexpr float kPfRescale = 8.0f;                   // lazy max threshold (log2 domain)
constexpr int kPfStageBlocks = 4;                    // blocks per pipeline stage
template <bool B>
struct PfF16 {  // a compile-time flag: the P.V operand type of a prefill pass, f16
                // (true) or bf16 high + residual, or whether a stage needs masks
  static constexpr bool value = B;
};

// LDS through address-space-3 pointers (ds_read / ds_write)
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ inline uint4 lds_ld16(const lds_u8* p) {
  return __builtin_bit_cast(uint4, *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p));
}
__device__ inline void lds_st16(lds_u8* p, uint4 x) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(p) = __builtin_bit_cast(u32x4, x);
}
__device__ inline void lds_st8(lds_u8* p, uint32_t x, uint32_t y) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(p) = u32x2{x, y};
}

// SB: blocks per pipeline stage (two pairs: P.V takes them in pairs).  F8: the
// cache holds FP8 E4M3 codes; each lane's 16 codes of a 1 KiB run are
// expanded to its two bf16 pieces on the way into LDS, so everything after
// the staging is the bf16 path (K scale folded into the score scale, V
// scale into out_scale).
template <int D, bool WIN, int SB, bool F8 = false>
__global__ __launch_bounds__(64 * kPfWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_bf16_kernel(PrefillArgs a) {
  static_assert(SB == 4, "a stage is two pairs of blocks");
  constexpr int NJ = D / 32;                  // K / V pieces per tile
  constexpr int NT = D / 16;                  // 16-channel output tiles
  constexpr int NQ = kPfColTiles;
  constexpr int TILE_BYTES = kBlock * D * 2;
  constexpr int STAGE_BYTES = 2 * SB * TILE_BYTES;  // blocks 0 .. SB-1 x (K, V)
  // tiles in global memory: as in LDS, or FP8 at one byte per element
  constexpr int TILE_G = F8 ? kBlock * D : TILE_BYTES;
  constexpr int TILE_PIECES_G = TILE_G / 16;
  constexpr int PT_G = 2 * SB * TILE_PIECES_G / (64 * kPfWaves);  // global pieces per thread
  static_assert(PT_G >= 1 && (2 * SB * TILE_PIECES_G) % (64 * kPfWaves) == 0,
                "a stage's global pieces spread evenly over the threads");
  constexpr int NBUF = 3;  // stage s, stage s + 1 (its first pair's scores), stage s + 2 being filled
  __shared__ __align__(16) unsigned char lds[NBUF * STAGE_BYTES];

  // Work item: workgroup i runs on XCD i % 8, and all query tiles of one
  // (sequence, kv head) pair run on one XCD, so they read its K/V through
  // one L2.  When the pairs are a multiple of 8, XCD x takes the pairs
  // p = x (mod 8) -- with 8 kv heads, head x of every sequence -- so every
  // XCD gets the same mix of context lengths; inside an XCD the longer items
  // go first, so the shorter ones fill in at the end.  Otherwise each XCD
  // takes a contiguous run of items.
  const int N = gridDim.x, id = blockIdx.x;
  const int npairs = a.num_seqs * a.num_kv_heads;
  int pair, qt;
  if (npairs % 8 == 0) {
    const int x = id % 8, j = id / 8;
    const int items = npairs / 8 * a.tiles;  // of this XCD: pairs x + 8 m, all tiles
    if (items <= 64) {
      // Longest first: lane i holds item i's stage count (the same arithmetic
      // as below), ranks by descending count with ties by index (a
      // permutation, identical in every workgroup), and this workgroup takes
      // the item of rank j.
      const int i = threadIdx.x & 63;
      int work = -1;
      if (i < items) {
        const int ib = (x + 8 * (i / a.tiles)) / a.num_kv_heads;
        const int iq0 = (i % a.tiles) * a.qtp;
        const int ins = a.qstart[ib], in = a.qstart[ib + 1] - ins, iL = a.lens[ib];
        work = 0;
        if (iq0 < in && in > 0 && iL >= in) {
          const int pf = iL - in + iq0, pl = pf + min(a.qtp, in - iq0) - 1;
          const int i0w = (WIN ? max(0, pf - a.window + 1) : 0) / kBlock;
          work = pl / kBlock + 1 - i0w;
        }
      }
      int rank = 0;
      for (int k = 0; k < items; ++k) {
        const int wk = __builtin_amdgcn_readlane(work, k);
        rank += (wk > work || (wk == work && k < i)) ? 1 : 0;
      }
      const int sel = static_cast<int>(__builtin_ctzll(
          __builtin_amdgcn_ballot_w64(i < items && rank == j)));
      pair = x + 8 * (sel / a.tiles);
      qt = sel % a.tiles;
    } else {
      pair = x + 8 * (j / a.tiles);
      qt = a.tiles - 1 - j % a.tiles;
    }
  } else {
    const int full = N / 8 * 8;
    const int w = id < full ? (id % 8) * (N / 8) + id / 8 : id;
    qt = w % a.tiles;
    pair = w / a.tiles;
  }
  const int kvh = pair % a.num_kv_heads;
  const int b = pair / a.num_kv_heads;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (kPfWaves - 1);
  const int hcol = lane & 15;
  const int grp = lane >> 4;
  const int g = a.group;
  const int QTP = a.qtp;
  const int qs = load_uniform(a.qstart, b);
  const int n = load_uniform(a.qstart, b + 1) - qs;
  const int q0 = qt * QTP;
  if (qt == a.tiles - 1 && n > a.tiles * QTP) {
    // chunk rows beyond the grid's tiles (max_query_len below this chunk):
    // NaN, so that no row of the output is left unwritten
    const int r0 = a.tiles * QTP;
    for (int c = wave; c < (n - r0) * g; c += kPfWaves) {
      float* dst = a.out + ((int64_t(qs) + r0 + c / g) * a.num_q_heads + int64_t(kvh) * g + c % g) * D;
      for (int e = lane; e < D; e += 64) dst[e] = __builtin_nanf("");
    }
  }
  if (q0 >= n || n <= 0) return;
  const int L = load_uniform(a.lens, b);
  const int nq = min(QTP, n - q0);  // positions in this tile
  const int ncol = nq * g;          // live columns
  auto out_row = [&](int c) -> float* {  // output row of column c
    return a.out + ((int64_t(qs) + q0 + c / g) * a.num_q_heads + int64_t(kvh) * g + c % g) * D;
  };
  const bool len_bad = L < 0 || L > a.max_ctx || int64_t(L) > int64_t(a.max_blocks) * kBlock ||
                       n > L;
  if (len_bad) {
    for (int c = wave; c < ncol; c += kPfWaves)
      for (int e = lane; e < D; e += 64) out_row(c)[e] = __builtin_nanf("");
    return;
  }
  const int p_first = L - n + q0;  // first and last position of the tile
  const int p_last = p_first + nq - 1;
  const int t_lo = WIN ? max(0, p_first - a.window + 1) : 0;  // earliest visible position
  const int i0 = t_lo / kBlock;
  const int nblk = p_last / kBlock + 1 - i0;
  const int nst = (nblk + SB - 1) / SB;
  const int32_t* row = a.tables + int64_t(b) * a.max_blocks + i0;

  // this lane's columns: c = 16 (NQ wave + t) + hcol -> (position, head)
  int pos[NQ], lo_c[NQ];
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    const int c = (NQ * wave + t) * 16 + hcol;
    pos[t] = c < ncol ? p_first + c / g : p_last;
    lo_c[t] = WIN ? pos[t] - a.window + 1 : 0;
  }

  // Q^T as B operands: lane holds q[row of column hcol][32j + 8 grp .. +8];
  // one resource over the tile's query rows, padding columns read past it (0)
  bf16x8 qf[NQ][NJ];
  {
    const int row_bytes = a.num_q_heads * D * 2;
    const char* qb = static_cast<const char*>(a.q) + (int64_t(qs) + q0) * row_bytes;
    const __amdgpu_buffer_rsrc_t rq = tile_rsrc(qb, nq * row_bytes);
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      const int c = (NQ * wave + t) * 16 + hcol;
      const int qoff = c < ncol ? (c / g) * row_bytes + (kvh * g + c % g) * D * 2 : nq * row_bytes;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        qf[t][j] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, qoff + (32 * j + grp * 8) * 2, 0, 0));
    }
  }

  const char* kc = static_cast<const char*>(a.kc) + int64_t(kvh) * TILE_G;
  const char* vc = static_cast<const char*>(a.vc) + int64_t(kvh) * TILE_G;
  const int64_t block_bytes = int64_t(a.num_kv_heads) * TILE_G;
  // a live block id outside the pool makes the tile's output NaN (its runs
  // load nothing)
  bool bad = false;
  for (int i = lane; i < nblk; i += 64)
    bad |= static_cast<unsigned>(row[i]) >= static_cast<unsigned>(a.num_blocks);
  bad = __builtin_amdgcn_ballot_w64(bad) != 0;

  // Stage loader.  A stage is SB blocks (tiles block 0 K, block 0 V, block
  // 1 K, ...), moved as 1 KiB runs (64 lanes x 16 bytes), each run by one
  // wavefront, so a run's tile and block id are wave-uniform: each run reads
  // its own block id through the scalar cache (reading the stage's entries
  // and selecting among them cost 3-6 % of the kernel in scalar work).  A
  // wavefront's runs are grouped in slots, the first half of them K and the
  // second V (with one slot per wavefront: the first four wavefronts K), so
  // the staging code has no branch on the tile kind.  bf16 cache: a slot is
  // the same 1 KiB piece of both blocks of a pair, so a lane holds both
  // halves of each P.V operand; FP8 cache: a slot is one run of codes, which
  // expands to two bf16 runs in LDS.  V slots outside [t_lo, L) are zeroed a
  // stage after their loads (they may hold anything; masking them at load
  // time would wait for the loads at once).
  uint4 st[PT_G];
  constexpr bool PAIRED = !F8;
  constexpr int RPT = TILE_PIECES_G / 64;        // runs per tile
  constexpr int PR = PAIRED ? 2 : 1;             // runs per slot
  constexpr int NS = PT_G / PR;                  // slots per wavefront
  constexpr int KIND = SB * RPT / PR;            // slots of K (and of V) per stage
  static_assert(PT_G % PR == 0 && (NS == 1 ? 2 * KIND == kPfWaves
                                           : NS % 2 == 0 && NS / 2 * kPfWaves == KIND),
                "a stage's slots spread evenly over the wavefronts, K and V apart");
  auto slot_v = [&](int i) { return NS == 1 ? wave >= kPfWaves / 2 : i >= NS / 2; };
  auto slot_k = [&](int i) {  // index among the stage's slots of its kind
    return NS == 1 ? wave % (kPfWaves / 2) : (i % (NS / 2)) * kPfWaves + wave;
  };
  // run u (slot u / PR): V or K, its block in the stage, its byte offset in the tile
  auto run_v = [&](int u) { return slot_v(u / PR); };
  auto run_blk = [&](int u) { return PR * (slot_k(u / PR) / RPT) + u % PR; };
  auto run_off = [&](int u) { return (slot_k(u / PR) % RPT) * 1024; };
  // The block ids of the stage the next gload takes, lane j holding entry
  // SB s + j (entries past the tile's last block read as 0 and go unused),
  // loaded one call ahead with a vector load: a run takes its id with a lane
  // read instead of a scalar-cache round trip (whose wait would also drain
  // the wavefront's LDS operations in flight).  Calls go 0, 1, 2, ... from
  // the start of each run.
  const __amdgpu_buffer_rsrc_t rrow = tile_rsrc(row, nblk * 4);
  auto idload = [&](int s) {
    return static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(rrow, (SB * s + (lane & (SB - 1))) * 4, 0, 0));
  };
  int idq = 0;
  auto gload = [&](int s) {
    const int ids = idq;
    idq = idload(s + 1);
#pragma unroll
    for (int u = 0; u < PT_G; ++u) {
      // this run's block id (wave-uniform); a run past the last block loads nothing
      const int rel = SB * s + run_blk(u);
      const bool live = rel < nblk;
      const int phys = __builtin_amdgcn_readlane(ids, run_blk(u));
      const bool use = live && static_cast<unsigned>(phys) < static_cast<unsigned>(a.num_blocks);
      const int off0 = run_off(u);
      // (an unused run points at block 0 with no bytes: selects, not branches)
      const uint32_t pid = use ? static_cast<uint32_t>(phys) : 0u;
      const __amdgpu_buffer_rsrc_t r =
          tile_rsrc((run_v(u) ? vc : kc) + int64_t(pid) * block_bytes + off0, use ? TILE_G - off0 : 0);
      st[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, 0, 0));
    }
  };
  // V slots of stage s outside [t_lo, L): lane l of a V run holds tokens
  // 4 (l / 16) .. + 3 of its block (16-bit fields t % 4 and 4 + t % 4 of
  // each 8-element piece; FP8: bytes).  Only a block that holds positions
  // before t_lo or from L on (tested once per block, wave-uniform) is masked.
  auto vmask = [&](int s) {
#pragma unroll
    for (int u = 0; u < PT_G; ++u) {
      const int b0 = (i0 + SB * s + run_blk(u)) * kBlock;
      if (run_v(u) && (b0 < t_lo || b0 + kBlock > L)) {
        const int t0 = b0 + 4 * grp;
        auto in = [&](int t) { return t < L && t >= t_lo; };
        uint4& x = st[u];
        if constexpr (F8) {
          const uint32_t mk = (in(t0) ? 0x000000FFu : 0u) | (in(t0 + 1) ? 0x0000FF00u : 0u) |
                              (in(t0 + 2) ? 0x00FF0000u : 0u) | (in(t0 + 3) ? 0xFF000000u : 0u);
          x.x &= mk;
          x.y &= mk;
          x.z &= mk;
          x.w &= mk;
        } else {
          const uint32_t m01 = (in(t0) ? 0x0000FFFFu : 0u) | (in(t0 + 1) ? 0xFFFF0000u : 0u);
          const uint32_t m23 = (in(t0 + 2) ? 0x0000FFFFu : 0u) | (in(t0 + 3) ? 0xFFFF0000u : 0u);
          x.x &= m01;
          x.y &= m23;
          x.z &= m01;
          x.w &= m23;
        }
      }
    }
  };
  // V tiles are stored in LDS as P.V reads them.  For the blocks 2p and
  // 2p + 1 of a stage, the tile slot of block 2p holds, at each 16-byte
  // chunk, the chunk's low 8 bytes of block 2p then those of block 2p + 1,
  // and the slot of block 2p + 1 the high 8 bytes of both, so each chunk is
  // one operand of the pair's product, read as it lies.  A bf16 lane holds
  // the same piece of both blocks and writes the two chunks whole; an FP8
  // run holds one block, written as 8-byte halves.
  // This lane's address in stage buffer s % NBUF plus a wave-uniform
  // offset, made opaque to the compiler: each access then adds its constant
  // tile offset as the instruction's immediate (from one visible base, the
  // three 32 KiB buffers lie beyond the immediate's 64 KiB reach and every
  // access took a vector add of its own).
  auto lbase = [&](int s, int extra) -> lds_u8* {
    uint32_t v = static_cast<uint32_t>((uintptr_t)(lds_u8*)lds) + (s % NBUF) * STAGE_BYTES + lane * 16 + extra;
    __asm__("" : "+v"(v));
    return (lds_u8*)(uintptr_t)v;
  };
  auto vstore = [&](lds_u8* sb, int blk, int o, uint4 x) {
    const int lo = (4 * (blk >> 1) + 1) * TILE_BYTES + o + 8 * (blk & 1);
    lds_st8(sb + lo, x.x, x.y);
    lds_st8(sb + lo + 2 * TILE_BYTES, x.z, x.w);
  };
  // stage s from the staging registers into its LDS buffer; V goes in as
  // f16 when P.V runs on f16 operands (H), where a bf16 V element with no
  // f16 equal becomes an f16 infinity or NaN
  auto lstore = [&](int s, auto h) {
    constexpr bool H = decltype(h)::value;
    lds_u8* sb = lbase(s, PAIRED ? run_off(0) : 2 * run_off(0));
    if constexpr (PAIRED) {
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        uint4 x0 = st[2 * i], x1 = st[2 * i + 1];
        const int blk = run_blk(2 * i);  // the pair's first block
        const int o = run_off(2 * i) - run_off(0);
        if (slot_v(i)) {
          if constexpr (H) {
            x0 = make_uint4(bf16x2_to_f16x2(x0.x), bf16x2_to_f16x2(x0.y), bf16x2_to_f16x2(x0.z),
                            bf16x2_to_f16x2(x0.w));
            x1 = make_uint4(bf16x2_to_f16x2(x1.x), bf16x2_to_f16x2(x1.y), bf16x2_to_f16x2(x1.z),
                            bf16x2_to_f16x2(x1.w));
          }
          // the pair's operand halves: low 8 bytes of both into block 2p's
          // slot, high 8 bytes of both into block 2p + 1's
          lds_st16(sb + (2 * blk + 1) * TILE_BYTES + o, make_uint4(x0.x, x0.y, x1.x, x1.y));
          lds_st16(sb + (2 * blk + 3) * TILE_BYTES + o, make_uint4(x0.z, x0.w, x1.z, x1.w));
        } else {
          lds_st16(sb + (2 * blk) * TILE_BYTES + o, x0);
          lds_st16(sb + (2 * blk + 2) * TILE_BYTES + o, x1);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < PT_G; ++u) {
        // FP8 run i of a tile holds operand pieces 2i and 2i + 1 of each
        // lane (E4M3 values are exact in both bf16 and f16)
        const uint4 w = st[u];
        const int blk = run_blk(u);
        const int o = 2 * (run_off(u) - run_off(0));
        if (run_v(u)) {
          const uint4 x = H ? e4m3x8_to_f16x8(w.x, w.y) : e4m3x8_to_bf16x8(w.x, w.y);
          const uint4 y = H ? e4m3x8_to_f16x8(w.z, w.w) : e4m3x8_to_bf16x8(w.z, w.w);
          vstore(sb, blk, o, x);
          vstore(sb, blk, o + 1024, y);
        } else {
          lds_st16(sb + 2 * blk * TILE_BYTES + o, e4m3x8_to_bf16x8(w.x, w.y));
          lds_st16(sb + 2 * blk * TILE_BYTES + o + 1024, e4m3x8_to_bf16x8(w.z, w.w));
        }
      }
    }
  };

  f32x4 o[NQ][NT];
  // running max per column (log2 domain, scaled; a finite floor, so that a
  // column with nothing visible yet gets weights exp2(-inf - floor) = 0),
  // and the normalisers: row sums of the same weights that P.V uses,
  // formed by the matrix cores (P times a column of ones) in the output
  // layout, so numerator and denominator share every rounding
  float m[NQ];
  f32x4 lacc[NQ];
  const f16x8 ones16 = __builtin_bit_cast(f16x8, make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u));
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
  // weights exp2(cs * s - m) with cs > 0: a negative scale negates Q
  // instead (exact in bf16), so the scaled max is the raw max times cs.  A
  // scale below the smallest normal float (zero included) is taken as that
  // smallest normal: every finite score (|s| < 2^40) times it is below
  // 2^-86, so every visible weight is exactly 1 either way, while a masked
  // score (-inf) keeps weight 0 (with cs = 0 it would give -inf * 0 = NaN).
  const float cs = fabsf(a.scale_log2e) < FLT_MIN ? FLT_MIN : fabsf(a.scale_log2e);
  if (a.scale_log2e < 0.f) {
#pragma unroll
    for (int t = 0; t < NQ; ++t)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        uint4 x = __builtin_bit_cast(uint4, qf[t][j]);
        x.x ^= 0x80008000u;
        x.y ^= 0x80008000u;
        x.z ^= 0x80008000u;
        x.w ^= 0x80008000u;
        qf[t][j] = __builtin_bit_cast(bf16x8, x);
      }
  }

  // The unit of work is a pair of blocks (32 tokens).  Pair q of stage s:
  // K tiles 4q and 4q + 2 of the stage's buffer, V (in operand order)
  // tiles 4q + 1 and 4q + 3.  Its scores: S^T tiles per column tile and block.
  typedef f32x4 Scores[NQ][2];
  auto qk = [&](const lds_u8* kb, Scores& S) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      bf16x8 kx[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        kx[j] = __builtin_bit_cast(bf16x8, lds_ld16(kb + 2 * bb * TILE_BYTES + 1024 * j));
#pragma unroll
      for (int t = 0; t < NQ; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kx[j], qf[t][j], acc, 0, 0, 0);
        S[t][bb] = acc;
      }
    }
  };
  // Masks of a stage's two pairs (edge: the stage reaches past the tile's
  // first position, or before its last column's window start; masked
  // scores become -inf) and the lazy max: it is raised only when a column's
  // max over the stage exceeds it by 2^8, which a lane sees from its own
  // scores (any lane of the column), so the reduction over the column's
  // four lanes and the rescale of the accumulators run only then (once per
  // stage: a second rescale site per loop trip made the compiler copy every
  // accumulator at each trip).  tb0: the stage's first position.
  auto smax = [&](Scores& S0, Scores& S1, int tb0, bool edge) {
    if (edge) {
#pragma unroll
      for (int t = 0; t < NQ; ++t)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tp = tb0 + bb * kBlock + grp * 4 + r;
            if (tp > pos[t] || tp < lo_c[t]) S0[t][bb][r] = -INFINITY;
            if (tp + 2 * kBlock > pos[t] || tp + 2 * kBlock < lo_c[t]) S1[t][bb][r] = -INFINITY;
          }
    }
    float ml[NQ];
    bool need = false;
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      // a chain of three-way maxima (a NaN score, from NaN inputs, makes the
      // column's output NaN either way)
      float x = max_nan(S0[t][0][0], S0[t][0][1]);
      x = max_nan(max_nan(x, S0[t][0][2]), S0[t][0][3]);
      x = max_nan(max_nan(x, S0[t][1][0]), S0[t][1][1]);
      x = max_nan(max_nan(x, S0[t][1][2]), S0[t][1][3]);
      x = max_nan(max_nan(x, S1[t][0][0]), S1[t][0][1]);
      x = max_nan(max_nan(x, S1[t][0][2]), S1[t][0][3]);
      x = max_nan(max_nan(x, S1[t][1][0]), S1[t][1][1]);
      ml[t] = max_nan(max_nan(x, S1[t][1][2]), S1[t][1][3]);
      need |= ml[t] * cs > m[t] + kPfRescale;
    }
    if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
      for (int t = 0; t < NQ; ++t) {
        const float mloc = group_max(ml[t]) * cs;
        const bool raise = mloc > m[t] + kPfRescale;
        const float alpha = raise ? __builtin_amdgcn_exp2f(m[t] - mloc) : 1.0f;
        m[t] = raise ? mloc : m[t];
        // output rows are columns 4 grp + r of the tile; their factors sit in lanes 4 grp + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ar = __shfl(alpha, grp * 4 + r);
          lacc[t][r] *= ar;
#pragma unroll
          for (int k = 0; k < NT; ++k) o[t][k][r] *= ar;
        }
      }
    }
  };
  // weights of a pair: f16 pairs (H), else bf16 high parts and residuals;
  // operand element i < 4 is row i of the first block, i >= 4 of the second
  // (a masked score, -inf, gives exp2(-inf) = 0)
  auto sexp = [&](const Scores& S, uint32_t (&ph)[NQ][4], uint32_t (&pl)[NQ][4], auto h) {
    constexpr bool H = decltype(h)::value;
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      float p[8];
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[4 * bb + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[t][bb][r], cs, -m[t]));
        }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (H)
          ph[t][i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{p[2 * i], p[2 * i + 1]}), f16x2));
        else
          split_bf16x2(p[2 * i], p[2 * i + 1], ph[t][i], pl[t][i]);
      }
    }
  };
  // O += P . V over a pair (vb: the pair's first V tile slot); each V piece
  // is read once and used by all column tiles
  auto pv = [&](const lds_u8* vb, const uint32_t (&ph)[NQ][4], const uint32_t (&pl)[NQ][4],
                auto h) {
    constexpr bool H = decltype(h)::value;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const uint4 vl = lds_ld16(vb + 1024 * j);
      const uint4 vh = lds_ld16(vb + 2 * TILE_BYTES + 1024 * j);
#pragma unroll
      for (int t = 0; t < NQ; ++t) {
        if constexpr (H) {
          const f16x8 p = __builtin_bit_cast(f16x8, make_uint4(ph[t][0], ph[t][1], ph[t][2], ph[t][3]));
          o[t][2 * j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(p, __builtin_bit_cast(f16x8, vl), o[t][2 * j], 0, 0, 0);
          o[t][2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(p, __builtin_bit_cast(f16x8, vh), o[t][2 * j + 1], 0, 0, 0);
        } else {
          const bf16x8 p = __builtin_bit_cast(bf16x8, make_uint4(ph[t][0], ph[t][1], ph[t][2], ph[t][3]));
          const bf16x8 q = __builtin_bit_cast(bf16x8, make_uint4(pl[t][0], pl[t][1], pl[t][2], pl[t][3]));
          const bf16x8 lo = __builtin_bit_cast(bf16x8, vl), hi = __builtin_bit_cast(bf16x8, vh);
          o[t][2 * j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p, lo, o[t][2 * j], 0, 0, 0);
          o[t][2 * j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q, lo, o[t][2 * j], 0, 0, 0);
          o[t][2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p, hi, o[t][2 * j + 1], 0, 0, 0);
          o[t][2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q, hi, o[t][2 * j + 1], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      if constexpr (H) {
        const f16x8 p = __builtin_bit_cast(f16x8, make_uint4(ph[t][0], ph[t][1], ph[t][2], ph[t][3]));
        lacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(p, ones16, lacc[t], 0, 0, 0);
      } else {
        const bf16x8 p = __builtin_bit_cast(bf16x8, make_uint4(ph[t][0], ph[t][1], ph[t][2], ph[t][3]));
        const bf16x8 q = __builtin_bit_cast(bf16x8, make_uint4(pl[t][0], pl[t][1], pl[t][2], pl[t][3]));
        lacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p, ones, lacc[t], 0, 0, 0);
        lacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q, ones, lacc[t], 0, 0, 0);
      }
    }
  };

  // One stage, software-pipelined: stage s + 2 from the staging registers
  // into its LDS buffer (its loads went out a stage earlier), the masks and
  // max of stage s's scores (both pairs, computed during the previous
  // stage), then per pair its weights with the scores of the same pair of
  // stage s + 1 issued among them (the products run on the matrix cores
  // while the vector unit works), then its P.V, the first among the loads of
  // stage s + 3.  S0, S1 hold the scores of stage s on entry, of stage s + 1
  // on exit.
  auto stage = [&](int s, Scores& S0, Scores& S1, auto h) {
    const lds_u8* cur = lbase(s, 0);
    const lds_u8* nxt = lbase(s + 1, 0);
    const int tb0 = (i0 + SB * s) * kBlock;
    // masks are needed only where the stage reaches past the tile's first
    // position (causal) or before its last column's window start
    const bool edge = tb0 + SB * kBlock - 1 > p_first || (WIN && tb0 < p_last - a.window + 1);
    uint32_t ph[NQ][4], pl[NQ][4];
    vmask(s + 2);
    lstore(s + 2, h);
    smax(S0, S1, tb0, edge);
    sexp(S0, ph, pl, h);
    qk(nxt, S0);
    pv(cur + TILE_BYTES, ph, pl, h);
    gload(s + 3);
    sexp(S1, ph, pl, h);
    qk(nxt + 4 * TILE_BYTES, S1);
    pv(cur + 5 * TILE_BYTES, ph, pl, h);
  };

  // Stage s is in LDS buffer s % 3.  The barrier at the top of stage s
  // makes stage s + 1 visible (written during stage s - 1; its scores are
  // taken during stage s) and frees buffer (s + 2) % 3 (every wavefront is
  // done with stage s - 1), which takes stage s + 2 from the staging
  // registers at the start of the stage; stage s + 3's loads go out after
  // the first pair's P.V.  Stages past the end load nothing and are stored
  // as zeros into buffers no wavefront is reading.
  auto run = [&](auto h) {
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
#pragma unroll
      for (int k = 0; k < NT; ++k) o[t][k] = f32x4{0.f, 0.f, 0.f, 0.f};
      m[t] = -1e30f;
      lacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    idq = idload(0);
    gload(0);
    vmask(0);
    lstore(0, h);
    gload(1);
    vmask(1);
    lstore(1, h);
    gload(2);
    __syncthreads();
    Scores S0, S1;
    qk(lbase(0, 0), S0);
    qk(lbase(0, 0) + 4 * TILE_BYTES, S1);
    for (int s = 0; s < nst; ++s) {
      if (s) __syncthreads();
      stage(s, S0, S1, h);
    }
  };
  // P.V on f16 operands: the weights lie in [0, 2^8] and round to 11
  // significant bits (bf16 would keep 8, and needs a residual product to
  // stay inside the tolerance).  A bf16 cache can hold V elements that f16
  // cannot (magnitude 2^16 and up, infinities, NaN); their f16 forms are
  // infinities or NaN, and the weight of every column times one of them
  // (weights are >= 0; 0 times infinity is NaN) leaves that accumulator
  // non-finite for the rest of the run, while finite operands cannot
  // overflow it (|o| < 2^8 * 65504 per position).  A workgroup with any
  // non-finite accumulator runs again with bf16 operands (the weights as
  // high part plus residual); so does one whose scores were NaN or infinite,
  // which then gives the same NaN output.
  run(PfF16<true>{});
  if constexpr (!F8) {
    float chk = 0.f;
#pragma unroll
    for (int t = 0; t < NQ; ++t)
#pragma unroll
      for (int k = 0; k < NT; ++k) chk += (o[t][k][0] + o[t][k][1]) + (o[t][k][2] + o[t][k][3]);
    __shared__ int s_wide[kPfWaves];
    const bool mine = __builtin_amdgcn_ballot_w64(!__builtin_isfinite(chk)) != 0;
    if (lane == 0) s_wide[wave] = mine;
    __syncthreads();  // also: every wavefront is done with the last stage's LDS
    int any = 0;
#pragma unroll
    for (int w = 0; w < kPfWaves; ++w) any |= s_wide[w];
    if (any) run(PfF16<false>{});
  }

#pragma unroll
  for (int t = 0; t < NQ; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int cl = grp * 4 + r;  // output row = column of the tile
      const int c = (NQ * wave + t) * 16 + cl;
      const float inv = bad ? __builtin_nanf("") : a.out_scale / lacc[t][r];
      if (c < ncol) {
        float* dst = out_row(c) + hcol;
#pragma unroll
        for (int k = 0; k < NT; ++k) dst[16 * k] = o[t][k][r] * inv;
      }
    }
  }
}

template <bool F8>
void launch_prefill_bf16(unsigned grid, hipStream_t stream, const PrefillArgs& a, int head_dim) {
  constexpr int SB = kPfStageBlocks;
  const dim3 block(64 * kPfWaves);
  const bool win = a.window > 0;
  if (head_dim == 64) {
    if (win)
      hipLaunchKernelGGL((prefill_bf16_kernel<64, true, SB, F8>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_bf16_kernel<64, false, SB, F8>), grid, block, 0, stream, a);
  } else if (win) {
    hipLaunchKernelGGL((prefill_bf16_kernel<128, true, SB, F8>), grid, block, 0, stream, a);
  } else {
    hipLaunchKernelGGL((prefill_bf16_kernel<128, false, SB, F8>), grid, block, 0, stream, a);
  }
}

}  // namespace

// ============================================================================ C ABI
namespace {
// Chunked prefill for a bf16 cache, or an FP8 one with tensor scales.
pkv_status prefill_impl(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* context_lens,
                        const int32_t* query_start, int32_t num_seqs, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                        int32_t max_blocks_per_seq, int32_t max_context_len,
                        int32_t max_query_len, float scale, int32_t window, bool fp8,
                        float k_scale, float v_scale, float* out, hipStream_t stream) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || max_context_len < 0 || max_query_len < 0 || window < 0)
    return PKV_ERR_INVALID;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_INVALID;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
  const int group = num_q_heads / num_kv_heads;
  if (group > 16) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0 || max_query_len == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start || !out)
    return PKV_ERR_INVALID;
  PrefillArgs a;
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.qstart = query_start;
  a.out = out;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.qtp = kPfCols / group;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.max_ctx = max_context_len;
  a.scale_log2e = scale * k_scale * 1.4426950408889634f;
  a.window = window;
  a.out_scale = v_scale;
  const int64_t tiles = (int64_t(max_query_len) + a.qtp - 1) / a.qtp;
  const int64_t grid = tiles * num_seqs * num_kv_heads;
  if (grid > 0x7FFFFFFF) return PKV_ERR_UNSUPPORTED;
  a.tiles = static_cast<int>(tiles);
  if (fp8)
    launch_prefill_bf16<true>(static_cast<unsigned>(grid), stream, a, head_dim);
  else
    launch_prefill_bf16<false>(static_cast<unsigned>(grid), stream, a, head_dim);
  return launch_status();
}
}  // namespace

extern "C" {

pkv_status paged_attention_prefill(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   const int32_t* query_start, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t num_blocks, int32_t max_blocks_per_seq,
                                   int32_t max_context_len, int32_t max_query_len, float scale,
                                   int32_t window, pkv_dtype kv_dtype, float* out,
                                   hipStream_t stream) {
  if (kv_dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  return prefill_impl(q, k_cache, v_cache, block_tables, context_lens, query_start, num_seqs,
                      num_q_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq,
                      max_context_len, max_query_len, scale, window, false, 1.0f, 1.0f, out,
                      stream);
}

pkv_status paged_attention_prefill_fp8(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, const int32_t* context_lens,
                                       const int32_t* query_start, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t num_blocks,
                                       int32_t max_blocks_per_seq, int32_t max_context_len,
                                       int32_t max_query_len, float scale, int32_t window,
                                       float k_scale, float v_scale, float* out,
                                       hipStream_t stream) {
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return PKV_ERR_INVALID;
  return prefill_impl(q, k_cache, v_cache, block_tables, context_lens, query_start, num_seqs,
                      num_q_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq,
                      max_context_len, max_query_len, scale, window, true, k_scale, v_scale, out,
                      stream);
}

}  // extern "C"
