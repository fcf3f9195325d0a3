// Device side of libpagedkv: HIP kernels for gfx950 (CDNA4) and the C ABI
// entry points that launch them.
//
// Kernels:
//   table_update      block-table (and length) deltas into device-resident tables
//   kv_write          scatter of new tokens' K/V through the slot mapping
//   append            table deltas and the scatter in one launch (a decode step)
//   kv_write_fp8      the scatter with E4M3 quantisation
//   copy_blocks       whole-block copies inside a cache (copy-on-write)
//   swap_blocks       whole-block copies between a cache and a pinned-host swap space
//   decode_bf16_cu    decode attention, default form: the block list split evenly
//                     over the CUs, partial states folded inside each CU and merged
//                     across CUs in the same launch; bf16 or FP8 cache, optional
//                     sliding window
//   decode_bf16_balanced  the same split per wavefront (fallback form)
//   decode_bf16 / decode_f32 + lse_reduce  fixed split-K partitions
//   stream_read       plain streaming read, the bandwidth reference
// (chunked prefill is in prefill.hip; shared helpers in device_common.h)
//
// Sources: "PagedAttention por dentro" (blog.lo0.es), sections "La tabla de
// paginas (block table)", "Copy-on-write para sampling paralelo", "El kernel
// CUDA" (attention walks the context in block-aligned chunks, each located
// through the table), "Chunked prefill integrado con paged KV", "Prefix
// caching cross-session", "Evicción y preemption" and "Sliding window
// attention"; "Como funciona realmente vLLM" (alexanderzelada.com), "Que es
// el mecanismo de atencion" and "PagedAttention: ..." (scattered blocks are
// read in place through the table, never gathered into a contiguous buffer);
// "KV cache: la memoria de trabajo..." (blog.lo0.es), «Trucos para que el
// cuaderno sea más fino» (an 8-bit cache).
//
// Matrix-core layout (bf16).  The cache tile order (pagedkv.h) makes lane l's
// 16-byte piece j of a tile exactly its matrix-core operand:
//   K piece j = 8 channels 32j + 8(l/16) .. +8 of token l%16
//       -> A operand of v_mfma_f32_16x16x32_bf16 (rows = tokens, k = channels)
//   V piece j = 4 tokens 4(l/16) .. +4 at channel 32j + l%16 (low half) and
//       channel 32j + 16 + l%16 (high half)
//       -> B operands of v_mfma_f32_16x16x16_bf16 (k = tokens, cols = channels)
// so each load instruction of a wavefront reads 1 KiB of contiguous memory
// and nothing is reshuffled.  Scores come out as S^T[token 4(l/16)+i][query
// head l%16] -- exactly the A-operand layout of the P.V product (rows =
// heads, k = tokens) -- so up to 16 query heads of a kv head share one pass
// over the tile.  In bf16 decode, softmax weights are split into a bf16 high
// part and a bf16 residual so that P.V keeps ~16 bits of weight precision;
// where V fits f16 (FP8 codes; the prefill's bf16 V below 65536) the weights
// and V enter P.V as f16 instead.  Accumulation is fp32 throughout.  An FP8 tile holds the same pieces at one byte per
// element, a lane's pieces paired into 16 bytes.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "device_common.h"
#include "pagedkv.h"

// The allocation-free decode's scratch (see scratch_device below).
static __device__ __align__(256) unsigned char scratch[size_t(16) << 20];

namespace {

// ------------------------------------------------------------------ A2: table deltas
__global__ void table_update_kernel(int32_t* __restrict__ tables, int64_t elems,
                                    const int32_t* __restrict__ upd, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int64_t idx = ld_sys(upd + 2 * i);
  if (idx >= 0 && idx < elems) tables[idx] = ld_sys(upd + 2 * i + 1);
}

// ------------------------------------------------------------------ A3: cache write
// One thread per (token, kv head, group of 8 channels).
template <typename T>
__global__ void kv_write_kernel(const T* __restrict__ k_new, const T* __restrict__ v_new,
                                const int64_t* __restrict__ slots, T* __restrict__ kc,
                                T* __restrict__ vc, int64_t total, int num_kv_heads, int head_dim,
                                int64_t num_slots) {
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int chunks = head_dim >> 3;
  const int c = static_cast<int>(idx % chunks);
  const int64_t ih = idx / chunks;
  const int h = static_cast<int>(ih % num_kv_heads);
  const int64_t i = ih / num_kv_heads;
  // the row chunk first: its loads and the slot's read (possibly over the
  // host link) are then in flight together
  const int64_t src = (i * num_kv_heads + h) * head_dim + c * 8;
  T kv[8], vv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    kv[e] = k_new[src + e];
    vv[e] = v_new[src + e];
  }
  const int64_t slot = ld_sys(slots + i);
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot >> 4;
  const int t = static_cast<int>(slot & 15);
  const int64_t tile = (blk * num_kv_heads + h) * int64_t(kBlock) * head_dim;
  // K: the 8 channels of a group are contiguous for a token
#pragma unroll
  for (int e = 0; e < 8; ++e) kc[tile + k_elem(t, c * 8 + e)] = kv[e];
#pragma unroll
  for (int e = 0; e < 8; ++e) vc[tile + v_elem(t, c * 8 + e)] = vv[e];
}

// ------------------------------------------------------------------ A2 + A3 fused
// Workgroups [0, table_wgs) apply table deltas; the rest scatter K/V rows
// to the same places as kv_write_kernel, with streaming stores.
template <typename T>
__global__ void append_kernel(const T* __restrict__ k_new, const T* __restrict__ v_new,
                              const int64_t* __restrict__ slots, T* __restrict__ kc,
                              T* __restrict__ vc, int64_t total, int num_kv_heads, int head_dim,
                              int64_t num_slots, int32_t* __restrict__ tables, int64_t elems,
                              const int32_t* __restrict__ upd, int n_upd, int table_wgs) {
  if (static_cast<int>(blockIdx.x) < table_wgs) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n_upd) {
      const int64_t idx = ld_sys(upd + 2 * i);
      if (idx >= 0 && idx < elems) tables[idx] = ld_sys(upd + 2 * i + 1);
    }
    return;
  }
  const int64_t idx = int64_t(blockIdx.x - table_wgs) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int chunks = head_dim >> 3;
  const int c = static_cast<int>(idx % chunks);
  const int64_t ih = idx / chunks;
  const int h = static_cast<int>(ih % num_kv_heads);
  const int64_t i = ih / num_kv_heads;
  // the row chunk first: its loads and the slot's read (possibly over the
  // host link) are then in flight together
  const int64_t src = (i * num_kv_heads + h) * head_dim + c * 8;
  T kv[8], vv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    kv[e] = k_new[src + e];
    vv[e] = v_new[src + e];
  }
  const int64_t slot = ld_sys(slots + i);
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot >> 4;
  const int t = static_cast<int>(slot & 15);
  const int64_t tile = (blk * num_kv_heads + h) * int64_t(kBlock) * head_dim;
  // Streaming stores: the rows are read again only by the next launch, and
  // lines left dirty in the L2 of each XCD slow that launch's start.
#pragma unroll
  for (int e = 0; e < 8; ++e)
    __builtin_nontemporal_store(kv[e], &kc[tile + k_elem(t, c * 8 + e)]);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    __builtin_nontemporal_store(vv[e], &vc[tile + v_elem(t, c * 8 + e)]);
}

// ------------------------------------------------------------------ A4: block copies
// blockIdx.x = pair, blockIdx.y = 0 (K) / 1 (V); a block of all heads is one
// contiguous run of `run16` 16-byte words.
__global__ void copy_blocks_kernel(uint4* __restrict__ kc, uint4* __restrict__ vc,
                                   const int32_t* __restrict__ pairs, int64_t run16,
                                   int num_blocks) {
  const int32_t src = ld_sys(pairs + 2 * blockIdx.x);
  const int32_t dst = ld_sys(pairs + 2 * blockIdx.x + 1);
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  uint4* base = blockIdx.y ? vc : kc;
  const uint4* s = base + int64_t(src) * run16;
  uint4* d = base + int64_t(dst) * run16;
  for (int64_t i = threadIdx.x; i < run16; i += blockDim.x) d[i] = s[i];
}

// ------------------------------------------------------------------ next: block swap
// Whole-block copies between two caches with the same block shape (the
// device cache and a swap space in pinned host memory, in either
// direction): pair i moves block pairs[i][0] of the source to block
// pairs[i][1] of the destination.  blockIdx.x = pair, blockIdx.y = 0 (K) /
// 1 (V).  Each lane keeps 4 loads in flight before their stores, so that
// the reads over the host link (long latency) overlap.
__global__ __launch_bounds__(256) void swap_blocks_kernel(
    const uint4* __restrict__ sk, const uint4* __restrict__ sv, uint4* __restrict__ dk,
    uint4* __restrict__ dv, const int32_t* __restrict__ pairs, int64_t run16, int src_blocks,
    int dst_blocks) {
  const int32_t src = ld_sys(pairs + 2 * blockIdx.x);
  const int32_t dst = ld_sys(pairs + 2 * blockIdx.x + 1);
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const uint4* s = (blockIdx.y ? sv : sk) + int64_t(src) * run16;
  uint4* d = (blockIdx.y ? dv : dk) + int64_t(dst) * run16;
  constexpr int U = 4;
  int64_t i = threadIdx.x;
  for (; i + (U - 1) * 256 < run16; i += U * 256) {
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = s[i + u * 256];
#pragma unroll
    for (int u = 0; u < U; ++u) d[i + u * 256] = w[u];
  }
  for (; i < run16; i += 256) d[i] = s[i];
}

// ------------------------------------------------------------------ A5: decode, bf16
struct DecodeArgs {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* tables;
  const int32_t* lens;
  float* out;
  float* ws_o;   // [B][Hq][max_parts][D]   unnormalised partial outputs
  float* ws_m;   // [B][Hq][max_parts]      running max (log2 domain)
  float* ws_l;   // [B][Hq][max_parts]      sum of weights
  int num_seqs, num_q_heads, num_kv_heads, group;
  int num_blocks, max_blocks, max_ctx, part_tokens, max_parts;
  float scale_log2e;
  // balanced mode: partial states of each wave's first (slot 0) and last
  // (slot 1) segment, [grid][2][group][D] and [grid][2][group]
  float* bw_o;
  float* bw_m;
  float* bw_l;
  unsigned long long* bw_count;  // [num_seqs * num_kv_heads]: epoch << 32 | arrivals
  unsigned epoch;                // distinct for every balanced launch
  int grid_waves;
  // per-CU form: overflow partial-state slots (over_slots per CU), fixed
  // share of each wavefront (per mille of the CU's range), minimum chunk
  // size in tiles
  float* cu_over;
  int over_slots;
  int static_permille, chunk_min;
  float out_scale;  // FP8 cache: the V tensor scale (1 otherwise)
  int window;       // sliding window in tokens (0: the whole context)
  // fused decode step (paged_kv_append_decode): each sequence with a context
  // gains the token of row s of k_new / v_new ([B][Hkv][D]); it is attended
  // from those rows and written to slots[s] at the end, with the table
  // deltas upd[n_upd][2] applied to tables_w[table_elems] and the new
  // lengths stored in lens_out (lens holds the lengths before the step)
  const void* k_new;
  const void* v_new;
  const int64_t* slots;
  int32_t* tables_w;
  int64_t table_elems;
  const int32_t* upd;
  int n_upd;
  int32_t* lens_out;
};

// Length check shared by the kernels: a bad length poisons the sequence.
__device__ inline bool len_ok(int L, const DecodeArgs& a) {
  return L >= 0 && L <= a.max_ctx && int64_t(L) <= int64_t(a.max_blocks) * kBlock;
}

// Sliding window: the query at position L-1 sees only the last `window`
// positions, [win_lo, L).  Blocks wholly before win_lo are never read (their
// table entries may already be released); the walk starts at the block
// holding win_lo and masks the positions before it.
// WIN = false compiles the window out (a kernel instance for window 0).
template <bool WIN = true>
__device__ inline int win_lo(const DecodeArgs& a, int L) {
  return (WIN && a.window > 0 && L > a.window) ? L - a.window : 0;
}
template <bool WIN = true>
__device__ inline int first_block_of(const DecodeArgs& a, int L) {
  return win_lo<WIN>(a, L) / kBlock;
}


// AUX is the cache policy of the K/V loads: 2 = non-temporal (the cache is
// streamed once per step; on MI355X this lifts the read rate by ~12 %),
// 0 = default, 18 = non-temporal + sc1.
template <int D, int ST, int AUX>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_bf16_kernel(DecodeArgs a) {
  constexpr int NJ = D / 32;  // 16-byte pieces per lane per tile (K and V each)
  constexpr int NT = D / 16;  // 16-channel output tiles
  constexpr int64_t TILE = int64_t(kBlock) * D;
  constexpr int TILE_BYTES = static_cast<int>(TILE * 2);

  const int lane = threadIdx.x;
  // 1D grid, kv head fastest: workgroup i runs on XCD i % 8, so each XCD gets
  // the same kv heads of every sequence and partition (an equal share of
  // the work for any length mix, and blocks shared between sequences are
  // read through one XCD's L2)
  const int64_t wid = blockIdx.x;
  const int kvh = static_cast<int>(wid % a.num_kv_heads);
  const int b = static_cast<int>((wid / a.num_kv_heads) % a.num_seqs);
  const int part = static_cast<int>(wid / (int64_t(a.num_kv_heads) * a.num_seqs));
  const int hcol = lane & 15;  // query head within the group (B/A operand column/row)
  const int grp = lane >> 4;   // lane group: tokens 4*grp .. 4*grp+3 of a block
  const int g = a.group;
  const int L = a.lens[b];
  const int64_t head0 = int64_t(b) * a.num_q_heads + int64_t(kvh) * g;

  if (!len_ok(L, a) || L == 0) {
    if (part == 0) {
      const float fill = (L == 0) ? 0.f : __builtin_nanf("");
      for (int e = lane; e < g * D; e += 64) a.out[head0 * D + e] = fill;
    }
    return;
  }
  // partitions tile [base, L), base = the window start rounded down to a block
  const int wlo = win_lo(a, L);
  const int base = wlo / kBlock * kBlock;
  const int nparts = (L - base + a.part_tokens - 1) / a.part_tokens;
  if (part >= nparts) return;
  const int t_begin = base + part * a.part_tokens;
  const int t_end = min(L, t_begin + a.part_tokens);
  const int nblk = (t_end - t_begin + kBlock - 1) / kBlock;
  const int32_t* row = a.tables + int64_t(b) * a.max_blocks + t_begin / kBlock;

  // Q^T as B operand: lane holds q[head hcol][32j + 8*grp .. +8]; padded heads are 0.
  const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                       (head0 + (hcol < g ? hcol : 0)) * D + grp * 8;
  bf16x8 qf[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    uint4 w = *reinterpret_cast<const uint4*>(qp + 32 * j);
    if (hcol >= g) w = make_uint4(0, 0, 0, 0);
    qf[j] = __builtin_bit_cast(bf16x8, w);
  }

  const char* kc = static_cast<const char*>(a.kc) + int64_t(kvh) * TILE_BYTES;
  const char* vc = static_cast<const char*>(a.vc) + int64_t(kvh) * TILE_BYTES;
  const int64_t block_bytes = int64_t(a.num_kv_heads) * TILE_BYTES;
  const int loff = lane * 16;

  f32x4 o[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;  // running max of this lane's head (log2 domain)
  float lsum = 0.f;     // this lane's share of the sum of weights
  bool bad = false;

  // physical block of partition block i (clamped into the partition; ids past
  // its end are fetched but never used for a live load)
  auto block_id = [&](int i) -> int {
    return __builtin_amdgcn_readfirstlane(row[min(i, nblk - 1)]);
  };
  auto issue = [&](int i, int phys, uint4 (&kr)[NJ], uint4 (&vr)[NJ]) {
    int bytes = TILE_BYTES;
    if (i >= nblk) {
      bytes = 0;
    } else if (phys < 0 || phys >= a.num_blocks) {
      bad = true;
      bytes = 0;
    }
    const int64_t off = int64_t(bytes ? phys : 0) * block_bytes;
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kc + off, bytes);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vc + off, bytes);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      kr[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, loff + 1024 * j, 0, AUX));
      vr[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, loff + 1024 * j, 0, AUX));
    }
  };

  auto compute_block = [&](int i, const uint4 (&kr)[NJ], uint4 (&vr)[NJ]) {
    // S^T = K . Q^T : lane holds tokens 4*grp+r (r = 0..3) for head hcol
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[j]), qf[j], s,
                                                   0, 0, 0);
    const int tb = t_begin + i * kBlock + grp * 4;
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      sv[r] = (tb + r < t_end && tb + r >= wlo) ? s[r] * a.scale_log2e : -INFINITY;
    float mloc = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mloc = group_max(mloc);
    const float mnew = fmaxf(m, mloc);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(sv[r] - mnew);
    lsum = lsum * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    m = mnew;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
      // output rows are heads 4*grp+r; fetch their factors from lanes 4*grp+r
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, grp * 4 + r);
#pragma unroll
        for (int n = 0; n < NT; ++n) o[n][r] *= ar;
      }
    }
    // P as A operand (rows = heads hcol, k = tokens 4*grp+r), high + residual
    uint32_t hi01, lo01, hi23, lo23;
    split_bf16x2(p[0], p[1], hi01, lo01);
    split_bf16x2(p[2], p[3], hi23, lo23);
    const s16x4 phi = __builtin_bit_cast(s16x4, make_uint2(hi01, hi23));
    const s16x4 plo = __builtin_bit_cast(s16x4, make_uint2(lo01, lo23));
    if (t_begin + i * kBlock + kBlock > t_end || t_begin + i * kBlock < wlo) {
      // partial block: zero V of slots outside [wlo, t_end) (they may hold NaN)
      auto in = [&](int t) { return t < t_end && t >= wlo; };
      const uint32_t m01 = (in(tb + 0) ? 0x0000FFFFu : 0u) | (in(tb + 1) ? 0xFFFF0000u : 0u);
      const uint32_t m23 = (in(tb + 2) ? 0x0000FFFFu : 0u) | (in(tb + 3) ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        vr[j].x &= m01;
        vr[j].y &= m23;
        vr[j].z &= m01;
        vr[j].w &= m23;
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const s16x4 v0 = __builtin_bit_cast(s16x4, make_uint2(vr[j].x, vr[j].y));
      const s16x4 v1 = __builtin_bit_cast(s16x4, make_uint2(vr[j].z, vr[j].w));
      o[2 * j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, v0, o[2 * j], 0, 0, 0);
      o[2 * j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, v0, o[2 * j], 0, 0, 0);
      o[2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, v1, o[2 * j + 1], 0, 0, 0);
      o[2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, v1, o[2 * j + 1], 0, 0, 0);
    }
  };

  // ST-stage pipeline: while block i is computed, blocks i+1 .. i+ST-1 are in
  // flight.  Every trip issues the same loads (past the end they are empty),
  // and block ids are fetched one trip ahead of the loads that use them.
  uint4 kr[ST][NJ], vr[ST][NJ];
  int ids[ST];
#pragma unroll
  for (int st = 0; st < ST; ++st) ids[st] = block_id(st);
#pragma unroll
  for (int st = 0; st < ST; ++st) issue(st, ids[st], kr[st], vr[st]);
  for (int i0 = 0; i0 < nblk; i0 += ST) {
#pragma unroll
    for (int st = 0; st < ST; ++st) ids[st] = block_id(i0 + ST + st);
#pragma unroll
    for (int st = 0; st < ST; ++st) {
      const int i = i0 + st;
      if (i < nblk) compute_block(i, kr[st], vr[st]);
      issue(i + ST, ids[st], kr[st], vr[st]);
    }
  }

  lsum = group_sum(lsum);
  if (nparts == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = grp * 4 + r;
      const float lr = __shfl(lsum, h);
      const float inv = bad ? __builtin_nanf("") : 1.0f / lr;
      if (h < g) {
        float* dst = a.out + (head0 + h) * D + hcol;
#pragma unroll
        for (int n = 0; n < NT; ++n) dst[16 * n] = o[n][r] * inv;
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = grp * 4 + r;
      if (h < g) {
        float* dst = a.ws_o + ((head0 + h) * a.max_parts + part) * D + hcol;
#pragma unroll
        for (int n = 0; n < NT; ++n) dst[16 * n] = o[n][r];
      }
    }
    if (lane < g) {
      const int64_t mi = (head0 + lane) * a.max_parts + part;
      a.ws_m[mi] = bad ? __builtin_nanf("") : m;
      a.ws_l[mi] = lsum;
    }
  }
}

// ------------------------------------------------------------------ A5: decode, bf16, balanced
// Work-balanced form of the same computation.  All (kv head, sequence,
// block) tiles form one list, kv head slowest, then sequence, then block;
// wave w of the grid takes an equal contiguous slice of it and walks the
// slice across sequence boundaries with the same stage pipeline (so there
// is no per-partition start-up and no ragged tail of unequal partitions).
// A sequence's blocks that fall entirely inside one wave are finished there
// (output written directly); at most the first and the last segment of a
// wave are partial, and their (o, m, l) states go to slots 0 and 1 of that
// wave for the merge kernel.

// Tiles of a sequence in the work list: its blocks from the window's first.
template <bool WIN = true>
__device__ inline int nblocks_of(const DecodeArgs& a, int L) {
  return len_ok(L, a) ? (L + kBlock - 1) / kBlock - first_block_of<WIN>(a, L) : 0;
}

// Sum over the wave, returned as a wave-uniform value (scalar register), so
// that everything derived from it (slice bounds, buffer resources) stays
// uniform.
__device__ inline int wave_sum_int(int x) {
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return __builtin_amdgcn_readfirstlane(x);
}

__device__ inline int64_t balanced_per_wave(int64_t G, int waves) {
  constexpr int64_t kMinBlocks = 8;
  const int64_t per = (G + waves - 1) / waves;
  return per < kMinBlocks ? kMinBlocks : per;
}

template <int D, int ST, int AUX>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_bf16_balanced_kernel(DecodeArgs a) {
  constexpr int NJ = D / 32;
  constexpr int NT = D / 16;
  constexpr int64_t TILE = int64_t(kBlock) * D;
  constexpr int TILE_BYTES = static_cast<int>(TILE * 2);

  const int lane = threadIdx.x;
  const int hcol = lane & 15;
  const int grp = lane >> 4;
  const int g = a.group;
  const int B = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  const int64_t wid = blockIdx.x;

  // Block counts per sequence, 4 sequences per lane and 256 per pass: the
  // total over all sequences, then the tile where this wave's slice starts
  // (kv head, then sequence by a prefix scan).  For up to 256 sequences the
  // lengths stay in registers, so the start costs one round of length loads.
  int lenv[4], cnt[4];
  auto load_counts = [&](int c) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int b = c + lane * 4 + k;
      lenv[k] = b < B ? a.lens[b] : 0;
      cnt[k] = b < B ? nblocks_of(a, lenv[k]) : 0;
    }
  };
  // wave w writes the rows of the sequences b = w (mod grid) that have no
  // work: zeros for an empty context, NaN for a bad length
  auto fill_empty = [&](int c) {
    for (int b = static_cast<int>(wid); b < B; b += gridDim.x) {
      if (b < c || b >= c + 256) continue;
      const int pos = (b - c) >> 2, k = (b - c) & 3;
      const int L = __builtin_amdgcn_readlane(k == 0 ? lenv[0] : k == 1 ? lenv[1] : k == 2 ? lenv[2] : lenv[3], pos);
      if (!len_ok(L, a) || L == 0) {
        const float fill = (L == 0) ? 0.f : __builtin_nanf("");
        for (int e = lane; e < a.num_q_heads * D; e += 64)
          a.out[int64_t(b) * a.num_q_heads * D + e] = fill;
      }
    }
  };
  auto lane_scan = [&](int x) {  // inclusive prefix over lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int up = __shfl_up(x, d);
      if (lane >= d) x += up;
    }
    return x;
  };
  int total = 0;
  for (int c = 0; c < B; c += 256) {
    load_counts(c);
    fill_empty(c);
    total += wave_sum_int(cnt[0] + cnt[1] + cnt[2] + cnt[3]);
  }
  const int64_t G = int64_t(total) * Hkv;
  const int64_t per = balanced_per_wave(G, a.grid_waves);
  const int64_t g0 = wid * per;
  if (g0 >= G) return;
  const int64_t g1 = min(g0 + per, G);

  int c_kvh = static_cast<int>(g0 / total);
  int rem = static_cast<int>(g0 - int64_t(c_kvh) * total);
  int c_b = 0, c_blk = 0, c_L = 0;
  for (int c = 0, base = 0; c < B; c += 256) {
    if (B > 256) load_counts(c);  // else still in registers from the total
    const int mine = cnt[0] + cnt[1] + cnt[2] + cnt[3];
    const int incl = lane_scan(mine);
    const int chunk_total = __builtin_amdgcn_readlane(incl, 63);
    if (rem < base + chunk_total) {
      const uint64_t hit = __builtin_amdgcn_ballot_w64(base + incl > rem);
      const int pos = static_cast<int>(__builtin_ctzll(hit));
      int r = rem - (base + __builtin_amdgcn_readlane(incl, pos) - __builtin_amdgcn_readlane(mine, pos));
      int k = 0;
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        const int nq = __builtin_amdgcn_readlane(cnt[q], pos);
        if (k == q && r >= nq) {
          r -= nq;
          k = q + 1;
        }
      }
      c_b = c + pos * 4 + k;
      c_blk = r;
      c_L = __builtin_amdgcn_readlane(
          k == 0 ? lenv[0] : k == 1 ? lenv[1] : k == 2 ? lenv[2] : lenv[3], pos);
      break;
    }
    base += chunk_total;
  }
  c_b = __builtin_amdgcn_readfirstlane(c_b);
  c_blk = __builtin_amdgcn_readfirstlane(c_blk);
  c_L = __builtin_amdgcn_readfirstlane(c_L);
  int c_nb = nblocks_of(a, c_L);

  // the load cursor starts where the compute cursor starts
  int l_kvh = c_kvh, l_b = c_b, l_blk = c_blk, l_L = c_L, l_nb = c_nb;
  auto advance = [&](int& kvh, int& b, int& blk, int& L, int& nb) {
    ++blk;
    while (blk >= nb) {  // skips empty sequences
      blk = 0;
      if (++b == B) {
        b = 0;
        if (++kvh == Hkv) {  // past the list: park (never used for a live load)
          kvh = 0;
          nb = 1 << 30;
          break;
        }
      }
      L = load_uniform(a.lens, b);
      nb = nblocks_of(a, L);
    }
  };

  const int64_t block_bytes = int64_t(Hkv) * TILE_BYTES;
  const int loff = lane * 16;
  const int qoff = (hcol * D + grp * 8) * 2;  // >= g*D*2 for padded heads: reads as 0
  const int qbytes = g * D * 2;

  // stage buffers: K, V and (for the first block of a segment) Q
  uint4 kr[ST][NJ], vr[ST][NJ], qr[ST][NJ];
  bool st_bad[ST];
  int64_t l_idx = g0;
  auto issue = [&](int st) {
    const bool live = l_idx < g1;
    int phys = load_uniform(a.tables, int64_t(l_b) * a.max_blocks +
                                          (live ? first_block_of(a, l_L) + l_blk : 0));
    bool bad = false;
    int bytes = live ? TILE_BYTES : 0;
    if (live && (phys < 0 || phys >= a.num_blocks)) {
      bad = true;
      bytes = 0;
    }
    const int64_t off = (bytes ? int64_t(phys) * block_bytes : 0) + int64_t(l_kvh) * TILE_BYTES;
    const char* kc = static_cast<const char*>(a.kc) + off;
    const char* vc = static_cast<const char*>(a.vc) + off;
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kc, bytes);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vc, bytes);
    const bool needq = live && (l_blk == 0 || l_idx == g0);
    const char* qb = static_cast<const char*>(a.q) +
                     (int64_t(l_b) * a.num_q_heads + int64_t(l_kvh) * g) * D * 2;
    const __amdgpu_buffer_rsrc_t rq = tile_rsrc(qb, needq ? qbytes : 0);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      kr[st][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, loff + 1024 * j, 0, AUX));
      vr[st][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, loff + 1024 * j, 0, AUX));
      qr[st][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, qoff + 64 * j, 0, 0));
    }
    st_bad[st] = bad;
    if (live) advance(l_kvh, l_b, l_blk, l_L, l_nb);
    ++l_idx;
  };

  bf16x8 qf[NJ];
  f32x4 o[NT];
  float m = -INFINITY, lsum = 0.f;
  bool seg_bad = false;
  int seg_first_blk = 0;
  int64_t seg_start_idx = g0;
  bool seg_is_first = true;  // the segment that starts the slice
  // partial segments left for the merge: item (b * Hkv + kvh), its start in
  // the tile list and its block count, per slot (-1: none).  Plain scalars,
  // not arrays: a runtime-indexed private array would be placed in LDS, whose
  // per-lane addressing reads the dispatch packet from host memory at start.
  int part_item0 = -1, part_item1 = -1;
  int64_t part_start0 = 0, part_start1 = 0;
  int part_nb0 = 0, part_nb1 = 0;

  auto end_segment = [&](bool complete) {
    const float lt = group_sum(lsum);
    const int64_t head0 = int64_t(c_b) * a.num_q_heads + int64_t(c_kvh) * g;
    if (complete) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = grp * 4 + r;
        const float lr = __shfl(lt, h);
        const float inv = seg_bad ? __builtin_nanf("") : 1.0f / lr;
        if (h < g) {
          float* dst = a.out + (head0 + h) * D + hcol;
#pragma unroll
          for (int n = 0; n < NT; ++n) dst[16 * n] = o[n][r] * inv;
        }
      }
    } else {
      // partial state for the merge, written with device-scope (relaxed
      // atomic) stores: the wave that merges may run on another XCD, whose
      // L2 is not coherent with this one
      const int sl = seg_is_first ? 0 : 1;
      const int64_t slot = wid * 2 + sl;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = grp * 4 + r;
        if (h < g) {
          float* dst = a.bw_o + (slot * g + h) * D + hcol;
#pragma unroll
          for (int n = 0; n < NT; ++n)
            __hip_atomic_store(dst + 16 * n, o[n][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      if (lane < g) {
        __hip_atomic_store(a.bw_m + slot * g + lane, seg_bad ? __builtin_nanf("") : m,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.bw_l + slot * g + lane, lt, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
      if (sl == 0) {
        part_item0 = c_b * Hkv + c_kvh;
        part_start0 = seg_start_idx - seg_first_blk;
        part_nb0 = c_nb;
      } else {
        part_item1 = c_b * Hkv + c_kvh;
        part_start1 = seg_start_idx - seg_first_blk;
        part_nb1 = c_nb;
      }
    }
    seg_is_first = false;
  };

  auto compute = [&](int st, int64_t idx) {
    if (c_blk == 0 || idx == g0) {  // a segment starts: its Q came with this block
#pragma unroll
      for (int j = 0; j < NJ; ++j) qf[j] = __builtin_bit_cast(bf16x8, qr[st][j]);
#pragma unroll
      for (int n = 0; n < NT; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
      m = -INFINITY;
      lsum = 0.f;
      seg_bad = false;
      seg_first_blk = c_blk;
      seg_start_idx = idx;
    }
    seg_bad |= st_bad[st];
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[st][j]), qf[j], s,
                                                   0, 0, 0);
    // block c_blk of the list is block c_first + c_blk of the sequence
    const int wlo = win_lo(a, c_L);
    const int c_first = wlo / kBlock;
    const int tb = (c_first + c_blk) * kBlock + grp * 4;
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      sv[r] = (tb + r < c_L && tb + r >= wlo) ? s[r] * a.scale_log2e : -INFINITY;
    float mloc = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mloc = group_max(mloc);
    const float mnew = fmaxf(m, mloc);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(sv[r] - mnew);
    lsum = lsum * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    m = mnew;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, grp * 4 + r);
#pragma unroll
        for (int n = 0; n < NT; ++n) o[n][r] *= ar;
      }
    }
    uint32_t hi01, lo01, hi23, lo23;
    split_bf16x2(p[0], p[1], hi01, lo01);
    split_bf16x2(p[2], p[3], hi23, lo23);
    const s16x4 phi = __builtin_bit_cast(s16x4, make_uint2(hi01, hi23));
    const s16x4 plo = __builtin_bit_cast(s16x4, make_uint2(lo01, lo23));
    if ((c_first + c_blk) * kBlock + kBlock > c_L || (c_first + c_blk) * kBlock < wlo) {
      // zero V of slots outside [wlo, c_L) (they may hold NaN)
      auto in = [&](int t) { return t < c_L && t >= wlo; };
      const uint32_t m01 = (in(tb + 0) ? 0x0000FFFFu : 0u) | (in(tb + 1) ? 0xFFFF0000u : 0u);
      const uint32_t m23 = (in(tb + 2) ? 0x0000FFFFu : 0u) | (in(tb + 3) ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        vr[st][j].x &= m01;
        vr[st][j].y &= m23;
        vr[st][j].z &= m01;
        vr[st][j].w &= m23;
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const s16x4 v0 = __builtin_bit_cast(s16x4, make_uint2(vr[st][j].x, vr[st][j].y));
      const s16x4 v1 = __builtin_bit_cast(s16x4, make_uint2(vr[st][j].z, vr[st][j].w));
      o[2 * j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, v0, o[2 * j], 0, 0, 0);
      o[2 * j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, v0, o[2 * j], 0, 0, 0);
      o[2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, v1, o[2 * j + 1], 0, 0, 0);
      o[2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, v1, o[2 * j + 1], 0, 0, 0);
    }
    const bool last_of_seq = (c_blk == c_nb - 1);
    if (last_of_seq || idx == g1 - 1) end_segment(last_of_seq && seg_first_blk == 0);
    if (idx + 1 < g1) advance(c_kvh, c_b, c_blk, c_L, c_nb);
  };

#pragma unroll
  for (int st = 0; st < ST; ++st) issue(st);
  for (int64_t i0 = g0; i0 < g1; i0 += ST) {
#pragma unroll
    for (int st = 0; st < ST; ++st) {
      const int64_t i = i0 + st;
      if (i < g1) compute(st, i);
      issue(st);
    }
  }

  // Partial segments: once this wave's device-scope stores of its partial
  // states have completed (vmcnt 0 -- the same ordering the compiler uses
  // for an agent-scope release of atomic data, without an L2 write-back,
  // since nothing here is left dirty in L2), count an arrival on the
  // sequence's counter; the wave that brings the count to the number of
  // waves sharing the sequence merges, reading the states with device-scope
  // loads (no L2 invalidate needed for them).
  if (part_item0 < 0 && part_item1 < 0) return;
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  for (int sl = 0; sl < 2; ++sl) {
    const int item = sl == 0 ? part_item0 : part_item1;
    if (item < 0) continue;
    const int64_t s0 = sl == 0 ? part_start0 : part_start1;
    const int nbs = sl == 0 ? part_nb0 : part_nb1;
    const int64_t w0 = s0 / per, w1 = (s0 + nbs - 1) / per;
    const unsigned need = static_cast<unsigned>(w1 - w0 + 1);
    unsigned arrived = 0;
    if (lane == 0) {
      unsigned long long* cp = a.bw_count + item;
      unsigned long long old = __hip_atomic_load(cp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      unsigned long long nv = 0;
      for (int tries = 0; tries < (1 << 20); ++tries) {
        nv = (unsigned(old >> 32) == a.epoch) ? old + 1
                                              : ((static_cast<unsigned long long>(a.epoch) << 32) | 1ull);
        if (__hip_atomic_compare_exchange_weak(cp, &old, nv, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT))
          break;
      }
      arrived = static_cast<unsigned>(nv);
    }
    arrived = __builtin_amdgcn_readlane(arrived, 0);
    if (arrived != need) continue;
    __asm__ volatile("" ::: "memory");
    // merge: slot 1 of w0 when w0's slice began before the sequence, else
    // slot 0; partial states are folded in batches of kMergeBatch waves
    // (all loads of a batch in flight together), with a running maximum
    const int b = item / Hkv, kvh = item % Hkv;
    const int64_t head0 = int64_t(b) * a.num_q_heads + int64_t(kvh) * g;
    const bool split = (64 % g) == 0;
    const int lanes_per_head = split ? 64 / g : 64;
    const int h_first = split ? lane / lanes_per_head : 0;
    const int h_step = split ? g : 1;
    const int sub = split ? lane % lanes_per_head : lane;
    const int nd = D / lanes_per_head;  // channels per lane (<= D / 4)
    constexpr int kMergeBatch = 4;
    constexpr int NDMAX = D / 4;
    for (int h = h_first; h < g; h += h_step) {
      float M = -INFINITY, den = 0.f;
      float acc[NDMAX];
#pragma unroll
      for (int k = 0; k < NDMAX; ++k) acc[k] = 0.f;
      bool bad = false;
      for (int64_t wb = w0; wb <= w1; wb += kMergeBatch) {
        float mv[kMergeBatch], lv[kMergeBatch], ov[kMergeBatch][NDMAX];
#pragma unroll
        for (int c = 0; c < kMergeBatch; ++c) {
          const int64_t w = wb + c;
          const bool live = w <= w1;
          const int64_t slot = w * 2 + ((w == w0 && w0 * per < s0) ? 1 : 0);
          const int64_t mi = live ? slot * g + h : 0;
          mv[c] = live ? __hip_atomic_load(a.bw_m + mi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                       : -INFINITY;
          lv[c] = live ? __hip_atomic_load(a.bw_l + mi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                       : 0.f;
#pragma unroll
          for (int k = 0; k < NDMAX; ++k)
            ov[c][k] = (live && k < nd)
                           ? __hip_atomic_load(a.bw_o + mi * D + sub + k * lanes_per_head,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                           : 0.f;
        }
        float mc = M;
#pragma unroll
        for (int c = 0; c < kMergeBatch; ++c) {
          bad |= (mv[c] != mv[c]);
          mc = fmaxf(mc, mv[c]);
        }
        const float keep = __builtin_amdgcn_exp2f(M - mc);
        den *= keep;
#pragma unroll
        for (int k = 0; k < NDMAX; ++k) acc[k] *= keep;
#pragma unroll
        for (int c = 0; c < kMergeBatch; ++c) {
          const float f = __builtin_amdgcn_exp2f(mv[c] - mc);
          den = fmaf(f, lv[c], den);
#pragma unroll
          for (int k = 0; k < NDMAX; ++k) acc[k] = fmaf(f, ov[c][k], acc[k]);
        }
        M = mc;
      }
      const float inv = bad ? __builtin_nanf("") : 1.0f / den;
#pragma unroll
      for (int k = 0; k < NDMAX; ++k)
        if (k < nd) a.out[(head0 + h) * D + sub + k * lanes_per_head] = acc[k] * inv;
    }
  }
}

// Byte offset in an FP8 tile of lane `lane`'s 8-byte piece `j` (the codes of
// its bf16 operand piece j).  Pieces 2i and 2i + 1 of all lanes fill bytes
// [1024 i, 1024 i + 1024) as 64 lanes x 16 bytes, so one 16-byte load per
// lane reads 1 KiB in order; a last piece without a partner (D / 32 odd)
// takes 64 lanes x 8 bytes.
__device__ inline int f8_piece(int lane, int j, int head_dim) {
  const bool paired = 2 * (j / 2) + 1 < head_dim / 32;
  return 1024 * (j / 2) + (paired ? 16 : 8) * lane + 8 * (j % 2);
}

// Encode y (already divided by the tensor scale) as the nearest E4M3 code,
// ties to the even mantissa; magnitudes from 448 up clamp to 448 (0x7E);
// NaN gives the NaN code 0x7F; the sign bit is kept (also for zero).
__device__ inline uint32_t f32_to_e4m3(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  if (a != a) return sign | 0x7Fu;
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0x1p-6f) return sign | static_cast<uint32_t>(__builtin_rintf(a * 512.0f));  // m * 2^-9
  uint32_t u = __float_as_uint(a);
  u += 0x7FFFFu + ((u >> 20) & 1u);  // round the mantissa to 3 bits, ties to even
  const uint32_t code = ((((u >> 23) & 0xFFu) - 120u) << 3) | ((u >> 20) & 7u);
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

// FP8 cache write: one thread per (token, kv head, group of 8 channels);
// the inputs (bf16 or fp32) are multiplied by the inverse tensor scales in
// float32 and encoded.  FP8 tile order (one byte per element): K byte
// (t, d) at f8_piece(16 ((d / 8) % 4) + t, d / 32) + d % 8; V byte (t, d) at
// f8_piece(16 (t / 4) + d % 16, d / 32) + ((d / 16) % 2) 4 + t % 4 -- the
// bf16 tile's lanes and pieces, with a lane's pieces paired into 16 bytes.
template <typename T>
__device__ inline float widen_in(T x);
template <>
__device__ inline float widen_in<uint16_t>(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }
template <>
__device__ inline float widen_in<float>(float x) { return x; }

template <typename T>
__global__ void kv_write_fp8_kernel(const T* __restrict__ k_new, const T* __restrict__ v_new,
                                    const int64_t* __restrict__ slots, uint8_t* __restrict__ kc,
                                    uint8_t* __restrict__ vc, int64_t total, int num_kv_heads,
                                    int head_dim, int64_t num_slots, float k_inv, float v_inv) {
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int chunks = head_dim >> 3;
  const int c = static_cast<int>(idx % chunks);
  const int64_t ih = idx / chunks;
  const int h = static_cast<int>(ih % num_kv_heads);
  const int64_t i = ih / num_kv_heads;
  const int64_t slot = ld_sys(slots + i);
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot >> 4;
  const int t = static_cast<int>(slot & 15);
  const int64_t src = (i * num_kv_heads + h) * head_dim + c * 8;
  const int64_t tile = (blk * num_kv_heads + h) * int64_t(kBlock) * head_dim;
  uint32_t kq[8], vq[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    kq[e] = f32_to_e4m3(widen_in<T>(k_new[src + e]) * k_inv);
    vq[e] = f32_to_e4m3(widen_in<T>(v_new[src + e]) * v_inv);
  }
  // K: the 8 channels of the group are the 8 bytes of one lane piece
  const int d0 = c * 8;
  uint8_t* kd = kc + tile + f8_piece(16 * ((d0 / 8) % 4) + t, d0 / 32, head_dim);
  *reinterpret_cast<uint2*>(kd) = make_uint2(kq[0] | (kq[1] << 8) | (kq[2] << 16) | (kq[3] << 24),
                                             kq[4] | (kq[5] << 8) | (kq[6] << 16) | (kq[7] << 24));
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = d0 + e;
    vc[tile + f8_piece(16 * (t / 4) + d % 16, d / 32, head_dim) + ((d / 16) % 2) * 4 + t % 4] =
        static_cast<uint8_t>(vq[e]);
  }
}

// ------------------------------------------------------------------ A5: decode, bf16, per-CU balanced
// The same tile list, split first into one contiguous range per compute
// unit (one workgroup of 8 wavefronts per CU, holding all of its LDS).
// Inside a CU the work adapts to how fast each wavefront is served: each
// wavefront starts with a fixed share of the CU's range, then the rest is
// handed out in chunks of C tiles claimed from a counter in LDS.  Partial
// segments (at unit boundaries) go to slots, in LDS while it lasts, then in
// a per-CU overflow area of the workspace; after a workgroup barrier the
// wavefronts fold the slots of each sequence: a sequence wholly inside the
// CU's range is finished there, one that crosses the range boundary leaves
// one partial state per CU in global memory, merged (as in the per-wave
// form) by the last CU to arrive.  Claims and slot grants are LDS atomics,
// so nothing in the walk waits on vector memory beyond its own loads.
constexpr int kCuWaves = 8;
constexpr int kCuLdsBytes = 160 * 1024;
constexpr int kCuChunksMax = 64;                           // chunks per CU
constexpr float kCuRescale = 8.0f;                         // lazy-max threshold (log2)
constexpr int kCuSlots = 2 * (kCuWaves + kCuChunksMax);    // partial segments per CU
constexpr int kCuHeaderBytes = 64 + kCuSlots * 3 * 4;      // counters + slot metadata
// With the whole range in fixed shares (and chunks of at least 4 tiles) a CU
// runs at most 8 shares plus 2 chunks of the under-8-tile remainder, each
// leaving at most 2 partial segments.
constexpr int kCuStaticSlots = 2 * (kCuWaves + 2);
constexpr int kCuStaticChunkMin = 4;
// Sequences the per-CU form takes: their block-count prefix sits in LDS.
constexpr int kCuMaxSeqs = 16384;

// Partial-state slots: m and l [slot][group], then o [slot][group][D].
__host__ __device__ inline int cu_state_floats(int group, int head_dim) {
  return group * (head_dim + 2);
}
// LDS bytes of the block-count prefix of num_seqs sequences ([num_seqs + 1] ints).
__host__ __device__ inline int cu_prefix_bytes(int num_seqs) {
  return ((num_seqs + 1) * 4 + 15) & ~15;
}
// Slots that fit in LDS next to the header and the prefix (the rest overflow).
__host__ __device__ inline int cu_lds_slots(int group, int head_dim, int num_seqs) {
  const int n = (kCuLdsBytes - kCuHeaderBytes - cu_prefix_bytes(num_seqs)) /
                (cu_state_floats(group, head_dim) * 4);
  return n > kCuSlots ? kCuSlots : (n < 0 ? 0 : n);
}

// F8: the cache holds FP8 E4M3 codes (tiles of 16 D bytes, converted to
// bf16 in registers; scales folded into the score scale and out_scale).
// WIN: sliding window on (a.window > 0); off, the window code compiles out.
template <int D, int ST, int AUX, bool F8 = false, bool WIN = false, bool STEP = false>
__global__ __launch_bounds__(64 * kCuWaves) __attribute__((amdgpu_waves_per_eu(2)))
void decode_bf16_cu_kernel(DecodeArgs a) {
  static_assert(!(STEP && F8), "the fused step takes bf16 caches");
  constexpr int NJ = D / 32;
  constexpr int NT = D / 16;
  constexpr int NJ8 = NJ / 2;  // 16-byte loads per lane per FP8 tile (K and V each)
  constexpr int64_t TILE = int64_t(kBlock) * D;
  constexpr int TILE_BYTES = static_cast<int>(TILE * (F8 ? 1 : 2));
  constexpr int NW = kCuWaves;

  __shared__ __align__(16) unsigned char smem[kCuLdsBytes];
  const int g = a.group;
  const int B = a.num_seqs;
  const int cap = cu_lds_slots(g, D, B);  // slots held in LDS
  int* hdr = reinterpret_cast<int*>(smem);
  int* s_item = hdr + 16;
  int* s_s0 = s_item + kCuSlots;
  int* s_nb = s_s0 + kCuSlots;
  // s_cum[b] = tiles of the sequences before b in the list, b = 0..B
  int* s_cum = reinterpret_cast<int*>(smem + kCuHeaderBytes);
  float* s_m = reinterpret_cast<float*>(smem + kCuHeaderBytes + cu_prefix_bytes(B));
  float* s_l = s_m + cap * g;
  float* s_o = s_l + cap * g;
  // overflow slots of this CU in the workspace, [m g][l g][o g*D] per slot.
  // LDS and global slots are accessed on separate branches, so each access
  // compiles to an LDS or a global instruction (a pointer that could be
  // either would become a flat access, which the compiler waits on with the
  // vector-memory counter).
  float* const o_base = a.cu_over + int64_t(blockIdx.x) * a.over_slots * cu_state_floats(g, D);

  const int lane = threadIdx.x & 63;
  // wave-uniform (scalar register): everything derived from it stays uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hcol = lane & 15;
  const int grp = lane >> 4;
  const int Hkv = a.num_kv_heads;
  const int wg = blockIdx.x;
  const int NWG = gridDim.x;

  // Context length seen by this launch: in the fused step every sequence
  // with a context holds one more token (its row of k_new / v_new).
  auto grown = [](int L) { return (STEP && L > 0) ? L + 1 : L; };
  int64_t step_slot = -1;
  int32_t step_idx = -1, step_val = 0;
  // Tile counts of the B sequences and their prefix, in LDS.  Thread i takes
  // sequences [i k, i k + k); the length loads go through a buffer resource
  // sized to the B lengths (reads past them return 0, i.e. no tiles).
  {
    const int tid = threadIdx.x;
    const int k = (B + 64 * NW - 1) / (64 * NW);
    const __amdgpu_buffer_rsrc_t rl = tile_rsrc(a.lens, B * 4);
    int part = 0;
    for (int j = 0; j < k; ++j)
      part += nblocks_of<WIN>(a, grown(__builtin_amdgcn_raw_buffer_load_b32(rl, (tid * k + j) * 4, 0, 0)));

    int incl = part;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int up = __shfl_up(incl, d);
      if (lane >= d) incl += up;
    }
    if (lane == 63) hdr[4 + wave] = incl;  // wave totals
    __syncthreads();
    int run = incl - part;
    int total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int t = hdr[4 + w];
      run += w < wave ? t : 0;
      total += t;
    }
    for (int j = 0; j < k; ++j) {
      const int b = tid * k + j;
      if (b < B) {
        s_cum[b] = run;
        run += nblocks_of<WIN>(a, grown(__builtin_amdgcn_raw_buffer_load_b32(rl, b * 4, 0, 0)));
      }
    }
    if (tid == 0) s_cum[B] = total;
  }
  // rows of sequences with no work: zeros for an empty context, NaN for a
  // bad length, spread over all wavefronts of the grid
  for (int b = wg * NW + wave; b < B; b += NWG * NW) {
    const int L = grown(load_uniform(a.lens, b));
    if (!len_ok(L, a) || L == 0) {
      const float fill = (L == 0) ? 0.f : __builtin_nanf("");
      for (int e = lane; e < a.num_q_heads * D; e += 64)
        a.out[int64_t(b) * a.num_q_heads * D + e] = fill;
    }
  }
  __syncthreads();
  const int total = __builtin_amdgcn_readfirstlane(s_cum[B]);
  const int G = total * Hkv;  // < 2^31 (checked on the host)

  // this CU's range, the fixed share of each wavefront and the chunk size
  const int pc = G > 0 ? (G + NWG - 1) / NWG : 1;
  const int R0 = min(wg * pc, G);
  const int R1 = min(R0 + pc, G);
  const int S = static_cast<int>((int64_t(R1 - R0) * a.static_permille / 1000) / NW);
  const int Rs = R0 + NW * S;
  int C = (R1 - Rs + kCuChunksMax - 1) / kCuChunksMax;
  if (C < a.chunk_min) C = a.chunk_min;
  if (threadIdx.x == 0) {
    hdr[0] = Rs;  // next unclaimed tile
    hdr[1] = 0;   // slots used
  }
  __syncthreads();

  // tile index -> (kv head, sequence, block, length, block count): the
  // sequence is the last b with s_cum[b] <= the tile's rank in its kv head's
  // list (s_cum is non-decreasing, s_cum[0] = 0 and s_cum[B] = total), found
  // by a 64-way search, one LDS read and one ballot per level
  auto locate = [&](int t, int& kvh, int& b, int& blk, int& L, int& nb) {
    kvh = t / total;
    const int rem = t - kvh * total;
    int lo = 0, span = B;  // the answer lies in [lo, lo + span)
    while (span > 64) {
      const int stride = (span + 63) >> 6;
      const int off = lane * stride;
      const int v = off < span ? s_cum[lo + off] : 0x7FFFFFFF;
      const uint64_t le = __builtin_amdgcn_ballot_w64(v <= rem);
      const int p = 63 - static_cast<int>(__builtin_clzll(le));
      lo += p * stride;
      span = min(stride, span - p * stride);
    }
    const int v = lane < span ? s_cum[lo + lane] : 0x7FFFFFFF;
    const uint64_t le = __builtin_amdgcn_ballot_w64(v <= rem);
    b = __builtin_amdgcn_readfirstlane(lo + 63 - static_cast<int>(__builtin_clzll(le)));
    blk = __builtin_amdgcn_readfirstlane(rem - s_cum[b]);
    L = grown(load_uniform(a.lens, b));
    nb = nblocks_of<WIN>(a, L);
  };
  auto advance = [&](int& kvh, int& b, int& blk, int& L, int& nb) {
    ++blk;
    while (blk >= nb) {  // skips empty sequences
      blk = 0;
      if (++b == B) {
        b = 0;
        if (++kvh == Hkv) {  // past the list: park (never used for a live load)
          kvh = 0;
          nb = 1 << 30;
          break;
        }
      }
      L = grown(load_uniform(a.lens, b));
      nb = nblocks_of<WIN>(a, L);
    }
  };
  // claims the next chunk of the CU's range: [s, e), empty when none is left
  auto claim = [&](int& s, int& e) {
    int cs = 0;
    if (lane == 0) cs = atomicAdd(&hdr[0], C);
    cs = __builtin_amdgcn_readfirstlane(cs);
    s = min(cs, R1);
    e = min(cs + C, R1);
  };

  // load cursor: the fixed share first (or a first claim when there is none)
  int l_us = R0 + wave * S, l_ue = R0 + (wave + 1) * S;
  if (S == 0) claim(l_us, l_ue);
  bool l_live = l_us < l_ue;
  int l_idx = l_us;
  int l_kvh = 0, l_b = 0, l_blk = 0, l_L = 0, l_nb = 1;
  if (l_live) locate(l_us, l_kvh, l_b, l_blk, l_L, l_nb);

  const int64_t block_bytes = int64_t(Hkv) * TILE_BYTES;
  const int loff = lane * 16;
  const int qoff = (hcol * D + grp * 8) * 2;  // >= g*D*2 for padded heads: reads as 0
  const int qbytes = g * D * 2;

  uint4 kr[ST][F8 ? NJ8 : NJ], vr[ST][F8 ? NJ8 : NJ], qr[ST][NJ];
  bool st_bad[ST], rec_live[ST], rec_first[ST], rec_last[ST], rec_new[ST];
  int rec_kvh[ST], rec_b[ST], rec_blk[ST], rec_L[ST], rec_nb[ST], rec_idx[ST];

  auto issue = [&](int st) {
    const bool live = l_live;
    rec_live[st] = live;
    rec_kvh[st] = l_kvh;
    rec_b[st] = l_b;
    rec_blk[st] = l_blk;
    rec_L[st] = l_L;
    rec_nb[st] = l_nb;
    rec_idx[st] = l_idx;
    rec_first[st] = l_idx == l_us;
    rec_last[st] = l_idx == l_ue - 1;
    // fused step: the sequence's last tile holds the new token, which is
    // taken from its k_new / v_new row; when it opens a new block, nothing
    // of that block is in the cache yet (nor its table entry)
    const bool newtok = STEP && live && l_blk == l_nb - 1;
    const bool fresh = newtok && (l_L - 1) % kBlock == 0;
    rec_new[st] = newtok;
    // without branches: a stage with no tile reads entry 0 of the tables
    // (always there) and loads nothing
    const bool want = live && !fresh;
    const int phys = load_uniform(a.tables, want ? int64_t(l_b) * a.max_blocks +
                                                       first_block_of<WIN>(a, l_L) + l_blk
                                                 : int64_t(0));
    const bool ok = static_cast<unsigned>(phys) < static_cast<unsigned>(a.num_blocks);
    const bool bad = want && !ok;
    const int bytes = (want && ok) ? TILE_BYTES : 0;
    const int64_t off = (bytes ? int64_t(static_cast<uint32_t>(phys)) * block_bytes : 0) +
                        int64_t(l_kvh) * TILE_BYTES;
    const char* kc = static_cast<const char*>(a.kc) + off;
    const char* vc = static_cast<const char*>(a.vc) + off;
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kc, bytes);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vc, bytes);
    const bool needq = live && (l_blk == 0 || l_idx == l_us);
    const char* qb = static_cast<const char*>(a.q) +
                     (int64_t(l_b) * a.num_q_heads + int64_t(l_kvh) * g) * D * 2;
    const __amdgpu_buffer_rsrc_t rq = tile_rsrc(qb, needq ? qbytes : 0);
    if constexpr (F8) {
#pragma unroll
      for (int j = 0; j < NJ8; ++j) {
        kr[st][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, loff + 1024 * j, 0, AUX));
        vr[st][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, loff + 1024 * j, 0, AUX));
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        qr[st][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, qoff + 64 * j, 0, 0));
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        kr[st][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, loff + 1024 * j, 0, AUX));
        vr[st][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, loff + 1024 * j, 0, AUX));
        qr[st][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, qoff + 64 * j, 0, 0));
      }
    }
    st_bad[st] = bad;
    if (live) {
      if (l_idx == l_ue - 1) {
        claim(l_us, l_ue);
        l_live = l_us < l_ue;
        l_idx = l_us;
        if (l_live) locate(l_us, l_kvh, l_b, l_blk, l_L, l_nb);
      } else {
        advance(l_kvh, l_b, l_blk, l_L, l_nb);
        ++l_idx;
      }
    }
  };

  bf16x8 qf[NJ];
  f32x4 o[NT];
  float m = -INFINITY, lsum = 0.f;
  bool seg_bad = false;
  int seg_first_blk = 0;
  int seg_start_idx = 0;

  auto end_segment = [&](bool complete, int c_b, int c_kvh, int c_nb) {
    const float lt = group_sum(lsum);
    if (complete) {
      const int64_t head0 = int64_t(c_b) * a.num_q_heads + int64_t(c_kvh) * g;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = grp * 4 + r;
        const float lr = __shfl(lt, h);
        const float inv = seg_bad ? __builtin_nanf("") : a.out_scale / lr;
        if (h < g) {
          float* dst = a.out + (head0 + h) * D + hcol;
#pragma unroll
          for (int n = 0; n < NT; ++n) dst[16 * n] = o[n][r] * inv;
        }
      }
    } else {
      // (at most 2 per unit and 8 + kCuChunksMax units per CU: the slot
      // index stays below kCuSlots)
      int slot = 0;
      if (lane == 0) slot = atomicAdd(&hdr[1], 1);
      slot = __builtin_amdgcn_readfirstlane(slot);
      const float mv = seg_bad ? __builtin_nanf("") : m;
      if (slot < cap) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int h = grp * 4 + r;
          if (h < g) {
#pragma unroll
            for (int n = 0; n < NT; ++n) s_o[(slot * g + h) * D + hcol + 16 * n] = o[n][r];
          }
        }
        if (lane < g) {
          s_m[slot * g + lane] = mv;
          s_l[slot * g + lane] = lt;
        }
      } else {
        float* const base = o_base + (slot - cap) * cu_state_floats(g, D);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int h = grp * 4 + r;
          if (h < g) {
#pragma unroll
            for (int n = 0; n < NT; ++n) base[2 * g + h * D + hcol + 16 * n] = o[n][r];
          }
        }
        if (lane < g) {
          base[lane] = mv;
          base[g + lane] = lt;
        }
      }
      if (lane == 0) {
        s_item[slot] = c_b * Hkv + c_kvh;
        s_s0[slot] = seg_start_idx - seg_first_blk;
        s_nb[slot] = c_nb;
      }
    }
  };

  auto compute = [&](int st) {
    const int c_blk = rec_blk[st], c_L = rec_L[st], c_nb = rec_nb[st];
    if (c_blk == 0 || rec_first[st]) {  // a segment starts: its Q came with this block
#pragma unroll
      for (int j = 0; j < NJ; ++j) qf[j] = __builtin_bit_cast(bf16x8, qr[st][j]);
#pragma unroll
      for (int n = 0; n < NT; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
      m = -INFINITY;
      lsum = 0.f;
      seg_bad = false;
      seg_first_blk = c_blk;
      seg_start_idx = rec_idx[st];
    }
    seg_bad |= st_bad[st];
    // the stage's K and V as bf16 operand pieces
    uint4 kx[NJ], vx[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if constexpr (F8) {
        const uint4 kw = kr[st][j / 2], vw = vr[st][j / 2];
        kx[j] = (j & 1) ? e4m3x8_to_bf16x8(kw.z, kw.w) : e4m3x8_to_bf16x8(kw.x, kw.y);
        vx[j] = (j & 1) ? e4m3x8_to_f16x8(vw.z, vw.w) : e4m3x8_to_f16x8(vw.x, vw.y);
      } else {
        kx[j] = kr[st][j];
        vx[j] = vr[st][j];
      }
    }
    if constexpr (STEP) {
      if (rec_new[st]) {
        // the new token (slot tn of this tile) from its rows: K lanes l with
        // l % 16 == tn take channels 32 j + 8 (l / 16) .. + 8; V lanes with
        // l / 16 == tn / 4 take channels 32 j + l % 16 and 32 j + 16 + l % 16
        // into 16-bit field tn % 4 of their low and high halves
        const int tn = (c_L - 1) % kBlock;
        const int64_t row = (int64_t(rec_b[st]) * Hkv + rec_kvh[st]) * D;
        const uint16_t* kn = static_cast<const uint16_t*>(a.k_new) + row;
        const uint16_t* vn = static_cast<const uint16_t*>(a.v_new) + row;
        const bool kl = hcol == tn, vl = grp == (tn >> 2);
        const int sh = (tn & 1) * 16;
        const uint32_t keep = 0xFFFF0000u >> sh;  // the other token's half
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const uint4 kp = *reinterpret_cast<const uint4*>(kn + 32 * j + 8 * grp);
          const uint32_t vlo = vn[32 * j + hcol], vhi = vn[32 * j + 16 + hcol];
          if (kl) kx[j] = kp;
          if (vl) {
            if (tn & 2) {
              vx[j].y = (vx[j].y & keep) | (vlo << sh);
              vx[j].w = (vx[j].w & keep) | (vhi << sh);
            } else {
              vx[j].x = (vx[j].x & keep) | (vlo << sh);
              vx[j].z = (vx[j].z & keep) | (vhi << sh);
            }
          }
        }
      }
    }
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kx[j]), qf[j], s,
                                                   0, 0, 0);
    // block c_blk of the list is block c_first + c_blk of the sequence
    const int wlo = win_lo<WIN>(a, c_L);
    const int c_first = wlo / kBlock;
    const int tb = (c_first + c_blk) * kBlock + grp * 4;
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      sv[r] = (tb + r < c_L && tb + r >= wlo) ? s[r] * a.scale_log2e : -INFINITY;
    float mloc = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mloc = group_max(mloc);
    // lazy reference: raised only when a tile's max exceeds it by more than
    // kCuRescale (log2 domain), so weights stay below 2^kCuRescale and most
    // tiles skip rescaling the accumulators; the ratios do not depend on the
    // reference, and the merges carry it with each partial state.  (Every
    // tile holds a visible token, so a segment's first tile sets it.)
    const bool raise = mloc > m + kCuRescale;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float alpha = raise ? __builtin_amdgcn_exp2f(m - mloc) : 1.0f;
      m = raise ? mloc : m;
      lsum *= alpha;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, grp * 4 + r);
#pragma unroll
        for (int n = 0; n < NT; ++n) o[n][r] *= ar;
      }
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(sv[r] - m);
    if constexpr (F8) {
      // weights rounded to f16 once: P.V and the normaliser use the same values
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = static_cast<float>(static_cast<_Float16>(p[r]));
    }
    lsum += (p[0] + p[1]) + (p[2] + p[3]);
    uint32_t hi01, lo01 = 0, hi23, lo23 = 0;
    if constexpr (F8) {
      hi01 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{p[0], p[1]}), f16x2));
      hi23 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{p[2], p[3]}), f16x2));
    } else {
      split_bf16x2(p[0], p[1], hi01, lo01);
      split_bf16x2(p[2], p[3], hi23, lo23);
    }
    const s16x4 phi = __builtin_bit_cast(s16x4, make_uint2(hi01, hi23));
    const s16x4 plo = __builtin_bit_cast(s16x4, make_uint2(lo01, lo23));
    if ((c_first + c_blk) * kBlock + kBlock > c_L || (c_first + c_blk) * kBlock < wlo) {
      // zero V of slots outside [wlo, c_L) (they may hold NaN)
      auto in = [&](int t) { return t < c_L && t >= wlo; };
      const uint32_t m01 = (in(tb + 0) ? 0x0000FFFFu : 0u) | (in(tb + 1) ? 0xFFFF0000u : 0u);
      const uint32_t m23 = (in(tb + 2) ? 0x0000FFFFu : 0u) | (in(tb + 3) ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        vx[j].x &= m01;
        vx[j].y &= m23;
        vx[j].z &= m01;
        vx[j].w &= m23;
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const s16x4 v0 = __builtin_bit_cast(s16x4, make_uint2(vx[j].x, vx[j].y));
      const s16x4 v1 = __builtin_bit_cast(s16x4, make_uint2(vx[j].z, vx[j].w));
      if constexpr (F8) {
        typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
        const f16x4 ph = __builtin_bit_cast(f16x4, phi);
        o[2 * j] = __builtin_amdgcn_mfma_f32_16x16x16f16(ph, __builtin_bit_cast(f16x4, v0), o[2 * j], 0, 0, 0);
        o[2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(ph, __builtin_bit_cast(f16x4, v1), o[2 * j + 1], 0, 0, 0);
        continue;
      }
      o[2 * j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, v0, o[2 * j], 0, 0, 0);
      o[2 * j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, v0, o[2 * j], 0, 0, 0);
      o[2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, v1, o[2 * j + 1], 0, 0, 0);
      o[2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, v1, o[2 * j + 1], 0, 0, 0);
    }
    const bool last_of_seq = (c_blk == c_nb - 1);
    if (last_of_seq || rec_last[st])
      end_segment(last_of_seq && seg_first_blk == 0, rec_b[st], rec_kvh[st], c_nb);
  };

  // Every trip issues every stage (a stage past the end issues zero-size
  // loads), so the number of loads in flight at each wait is the same on all
  // paths and the compiler's waits stay partial.  Stages are filled in tile
  // order, so a dead stage 0 means all stages are dead.
#pragma unroll
  for (int st = 0; st < ST; ++st) issue(st);
  while (rec_live[0]) {
#pragma unroll
    for (int st = 0; st < ST; ++st) {
      if (rec_live[st]) compute(st);
      issue(st);
    }
  }
  if constexpr (STEP) {
    // this workgroup's first new-token slot and table delta, possibly read
    // over the host link: issued after the walk (inside it, every load wait
    // of the walk would wait for them too) and before the wait below, which
    // then covers them together with the walk's last loads
    if (wg < B) step_slot = ld_sys(a.slots + wg);
    const int i = wg + NWG * static_cast<int>(threadIdx.x);
    if (i < a.n_upd) {
      step_idx = ld_sys(a.upd + 2 * int64_t(i));
      step_val = ld_sys(a.upd + 2 * int64_t(i) + 1);
    }
  }
  // overflow slots were written with plain stores by other wavefronts of
  // this workgroup: complete them before the barrier
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // fused step: the first new rows this workgroup stores at the end, read
  // now so that their latency overlaps the fold
  constexpr int kStepCh = D / 8;  // 8-channel chunks per row and kv head
  uint4 step_k = make_uint4(0, 0, 0, 0), step_v = make_uint4(0, 0, 0, 0);
  if constexpr (STEP) {
    const int i = threadIdx.x;
    if (wg < B && i < Hkv * kStepCh) {
      const int64_t src = (int64_t(wg) * Hkv + i / kStepCh) * D + (i % kStepCh) * 8;
      step_k = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k_new) + src);
      step_v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v_new) + src);
    }
  }

  // Fold the slots of each sequence.  Wavefront w leads the slots s = w
  // (mod 8) that are the first slot of their sequence; lane element k is
  // channel (64 k + lane) of the group's heads, head (64 k + lane) / D.
  const int nsl = hdr[1];
  const int nk = g * D / 64;
  // Partial states of other CUs are read with the agent-coherent cache policy
  // (sc1, as a device-scope relaxed atomic load is) but as plain buffer
  // loads, so that all of a partner's values are in flight together.
  constexpr int kSc1 = 16;
  const __amdgpu_buffer_rsrc_t r_bo = tile_rsrc(a.bw_o, 0x7FFFFFF0);
  const __amdgpu_buffer_rsrc_t r_bm = tile_rsrc(a.bw_m, 0x7FFFFFF0);
  const __amdgpu_buffer_rsrc_t r_bl = tile_rsrc(a.bw_l, 0x7FFFFFF0);
  // Two passes: items that cross the CU's range first (their cross-CU
  // exchange has the longest latency), then the rest.  The fold runs once
  // per wavefront, at the end, from a cold instruction cache: its loops are
  // rolled over groups of 8 elements (unrolled inside for independent loads)
  // so that the same short code serves every group, slot and partner.
  for (int pass = 0; pass < 2; ++pass)
  for (int s = wave; s < nsl; s += NW) {
    const int item = s_item[s];
    const int s0 = s_s0[s], nbs = s_nb[s];
    const bool cross_start = s0 < R0, cross_end = s0 + nbs > R1;
    const bool crossing = cross_start || cross_end;
    if (crossing != (pass == 0)) continue;
    bool dup = false;
    for (int j0 = 0; j0 < s && !dup; j0 += 64) {
      const int j = j0 + lane;
      dup = __builtin_amdgcn_ballot_w64(j < s && s_item[j] == item) != 0;
    }
    if (dup) continue;
    // the item's slots from s on (slot indices below kCuSlots: 3 masks)
    const int c0 = s & ~63;
    uint64_t msk[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      const int jl = c0 + 64 * c + lane;
      msk[c] = __builtin_amdgcn_ballot_w64(jl >= s && jl < nsl && s_item[jl] == item);
    }
    const int b = item / Hkv, kvh = item % Hkv;
    const int64_t head0 = int64_t(b) * a.num_q_heads + int64_t(kvh) * g;
    // this CU's share of a crossing item goes to slot 0 when the item begins
    // at or before the range start, else slot 1
    const int64_t slot = int64_t(wg) * 2 + (s0 <= R0 ? 0 : 1);
    bool bad = false;
#pragma unroll 1
    for (int k0 = 0; k0 < nk; k0 += 8) {
      float acc[8], M[8], den[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc[u] = 0.f;
        M[u] = -INFINITY;
        den[u] = 0.f;
      }
#pragma unroll 1
      for (int c = 0; c < 3; ++c) {
        uint64_t mk = msk[c];
        while (mk) {
          const int j = c0 + 64 * c + static_cast<int>(__builtin_ctzll(mk));
          mk &= mk - 1;
          float mj[8], lj[8], oj[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int k = k0 + u < nk ? k0 + u : nk - 1;
            const int e = 64 * k + lane;
            const int h = (64 * k) / D;
            if (j < cap) {
              mj[u] = s_m[j * g + h];
              lj[u] = s_l[j * g + h];
              oj[u] = s_o[j * g * D + e];
            } else {
              const float* base = o_base + (j - cap) * cu_state_floats(g, D);
              mj[u] = base[h];
              lj[u] = base[g + h];
              oj[u] = base[2 * g + e];
            }
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            bad |= (mj[u] != mj[u]);
            const float mn = fmaxf(M[u], mj[u]);
            const float fo = __builtin_amdgcn_exp2f(M[u] - mn);
            const float fn = __builtin_amdgcn_exp2f(mj[u] - mn);
            acc[u] = acc[u] * fo + oj[u] * fn;
            den[u] = den[u] * fo + lj[u] * fn;
            M[u] = mn;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k0 + u;
        if (k < nk) {
          const int e = 64 * k + lane;
          const int h = (64 * k) / D;
          if (!crossing) {
            a.out[head0 * D + e] = bad ? __builtin_nanf("") : acc[u] / den[u] * a.out_scale;
          } else {
            __hip_atomic_store(a.bw_o + slot * g * D + e, acc[u], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            if ((e % D) == 0) {
              __hip_atomic_store(a.bw_m + slot * g + h, bad ? __builtin_nanf("") : M[u],
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              __hip_atomic_store(a.bw_l + slot * g + h, den[u], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
      }
    }
    if (!crossing) continue;
    // once the stores have completed, count this CU's arrival
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // arrival: the CU that brings the count to the number of CU ranges
    // covering the sequence merges their partial states
    const int w0 = s0 / pc, w1 = (s0 + nbs - 1) / pc;
    const unsigned need = static_cast<unsigned>(w1 - w0 + 1);
    unsigned arrived = 0;
    if (lane == 0) {
      unsigned long long* cp = a.bw_count + item;
      unsigned long long old = __hip_atomic_load(cp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      arrived = 0xFFFFFFFFu;  // stays so if the count could not be raised
      for (int tries = 0; tries < (1 << 20); ++tries) {
        const unsigned long long nv =
            (unsigned(old >> 32) == a.epoch)
                ? old + 1
                : ((static_cast<unsigned long long>(a.epoch) << 32) | 1ull);
        if (__hip_atomic_compare_exchange_weak(cp, &old, nv, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)) {
          arrived = static_cast<unsigned>(nv);
          break;
        }
      }
    }
    arrived = __builtin_amdgcn_readlane(arrived, 0);
    if (arrived == 0xFFFFFFFFu) {
      // this CU's arrival was never counted, so no CU will merge the item:
      // its rows become NaN rather than stay unwritten
      for (int e = lane; e < g * D; e += 64) a.out[head0 * D + e] = __builtin_nanf("");
      continue;
    }
    if (arrived != need) continue;
    __asm__ volatile("" ::: "memory");
    // merge every CU's share (this one's included, read back like the
    // others): each partner's 8 elements of a group in one round of loads
    bool gbad = false;
#pragma unroll 1
    for (int k0 = 0; k0 < nk; k0 += 8) {
      float acc[8], M[8], den[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc[u] = 0.f;
        M[u] = -INFINITY;
        den[u] = 0.f;
      }
#pragma unroll 1
      for (int w = w0; w <= w1; ++w) {
        const int gs = w * 2 + ((w == w0 && int64_t(w0) * pc < s0) ? 1 : 0);
        float mj[8], lj[8], oj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int k = k0 + u < nk ? k0 + u : nk - 1;
          const int e = 64 * k + lane;
          const int h = (64 * k) / D;
          oj[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_bo, (gs * g * D + e) * 4, 0, kSc1));
          mj[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_bm, (gs * g + h) * 4, 0, kSc1));
          lj[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_bl, (gs * g + h) * 4, 0, kSc1));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          gbad |= (mj[u] != mj[u]);
          const float mn = fmaxf(M[u], mj[u]);
          const float fo = __builtin_amdgcn_exp2f(M[u] - mn);
          const float fn = __builtin_amdgcn_exp2f(mj[u] - mn);
          acc[u] = acc[u] * fo + oj[u] * fn;
          den[u] = den[u] * fo + lj[u] * fn;
          M[u] = mn;
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (k0 + u < nk)
          a.out[head0 * D + 64 * (k0 + u) + lane] = gbad ? __builtin_nanf("") : acc[u] / den[u] * a.out_scale;
    }
  }

  if constexpr (STEP) {
    // The step's cache updates, on which nothing in this launch depends
    // (other workgroups may still be walking: a tile read after a row landed
    // has that token's bytes replaced from the rows all the same, the walk
    // skips the table entry of a block the new token opens, a copy-on-write
    // entry changes to a copy of the same bytes, and a released block lies
    // outside the window): every sequence s = wg, wg + NWG, ... with a
    // context stores its new K/V row in its slot (as paged_kv_write: slots
    // outside the pool are skipped), table deltas i = wg + NWG t are
    // applied, and the new lengths go to lens_out.
    const int tid = threadIdx.x;
    constexpr int CH = kStepCh;
    for (int sq = wg; sq < B; sq += NWG) {
      const int L0 = load_uniform(a.lens, sq);
      if (tid == 0) a.lens_out[sq] = grown(L0);
      const int64_t slot = sq == wg ? step_slot : ld_sys(a.slots + sq);
      if (!(L0 > 0) || slot < 0 || slot >= int64_t(a.num_blocks) * kBlock) continue;
      const int64_t blk = slot >> 4;
      const int t = static_cast<int>(slot & 15);
      for (int i = tid; i < Hkv * CH; i += 64 * NW) {
        const int h = i / CH, c = i % CH;
        const int64_t src = (int64_t(sq) * Hkv + h) * D + c * 8;
        const int64_t tile = (blk * Hkv + h) * int64_t(kBlock) * D;
        const bool pre = sq == wg && i == tid;  // read after the main loop
        const uint4 kw = pre ? step_k : *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k_new) + src);
        const uint4 vw = pre ? step_v : *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v_new) + src);
        uint16_t* kc = static_cast<uint16_t*>(const_cast<void*>(a.kc)) + tile;
        uint16_t* vc = static_cast<uint16_t*>(const_cast<void*>(a.vc)) + tile;
        const uint16_t ve[8] = {uint16_t(vw.x), uint16_t(vw.x >> 16), uint16_t(vw.y), uint16_t(vw.y >> 16),
                                uint16_t(vw.z), uint16_t(vw.z >> 16), uint16_t(vw.w), uint16_t(vw.w >> 16)};
        // K: the 8 channels of a group are 16 contiguous bytes for a token
        *reinterpret_cast<uint4*>(kc + k_elem(t, c * 8)) = kw;
#pragma unroll
        for (int e = 0; e < 8; ++e) vc[v_elem(t, c * 8 + e)] = ve[e];
      }
    }
    for (int i = wg + NWG * tid, r = 0; i < a.n_upd; i += NWG * 64 * NW, ++r) {
      const int32_t idx = r == 0 ? step_idx : ld_sys(a.upd + 2 * int64_t(i));
      const int32_t val = r == 0 ? step_val : ld_sys(a.upd + 2 * int64_t(i) + 1);
      if (idx >= 0 && idx < a.table_elems) a.tables_w[idx] = val;
    }
  }
}

// ------------------------------------------------------------------ A5: decode, fp32
// One wave per (sequence, query head, partition), a block (16 tokens) per
// step, the next block's id and K/V loads in flight during this one.
// Scores: lane (t, c) = (lane % 16, lane / 16) takes token t's dot product
// over the channel quarter c (D / 4 channels: runs of 8 in the tile order),
// the four quarters summed across lanes.  The block's max and weight sum are
// reductions over the 16 token lanes; the running max and normaliser are
// the online softmax applied once per block.  P.V: lane = channel (and
// channel + 64), its V values of the block are 4 runs of 4 tokens in the
// tile order, each weight read from its token's lane.  Plain vector-ALU
// form for the fp32 cache.
template <int D>
__global__ __launch_bounds__(64) void decode_f32_kernel(DecodeArgs a) {
  constexpr int NE = D / 64;     // output channels per lane
  constexpr int CQ = D / 4;      // channels per score lane
  constexpr int NR = CQ / 8;     // runs of 8 channels per score lane
  constexpr int64_t TILE = int64_t(kBlock) * D;
  const int lane = threadIdx.x;
  const int tok = lane & 15;
  const int cq = lane >> 4;
  const int64_t wid = blockIdx.x;  // query head fastest, then sequence, then partition
  const int hq = static_cast<int>(wid % a.num_q_heads);
  const int b = static_cast<int>((wid / a.num_q_heads) % a.num_seqs);
  const int part = static_cast<int>(wid / (int64_t(a.num_q_heads) * a.num_seqs));
  const int kvh = hq / a.group;
  const int L = a.lens[b];
  const int64_t head = int64_t(b) * a.num_q_heads + hq;
  if (!len_ok(L, a) || L == 0) {
    if (part == 0) {
      const float fill = (L == 0) ? 0.f : __builtin_nanf("");
      for (int e = lane; e < D; e += 64) a.out[head * D + e] = fill;
    }
    return;
  }
  // partitions tile [base, L), base = the window start rounded down to a block
  const int wlo = win_lo(a, L);
  const int base = wlo / kBlock * kBlock;
  const int nparts = (L - base + a.part_tokens - 1) / a.part_tokens;
  if (part >= nparts) return;
  const int t_lo = max(base + part * a.part_tokens, wlo);  // visible positions [t_lo, t_hi)
  const int t_hi = min(L, base + part * a.part_tokens + a.part_tokens);
  const int blk0 = t_lo / kBlock, blk1 = (t_hi - 1) / kBlock;  // blocks visited
  const int32_t* row = a.tables + int64_t(b) * a.max_blocks;
  const float* q = static_cast<const float*>(a.q) + head * D;
  const float* kc = static_cast<const float*>(a.kc) + kvh * TILE;
  const float* vc = static_cast<const float*>(a.vc) + kvh * TILE;
  const int64_t block_stride = int64_t(a.num_kv_heads) * TILE;
  // this lane's query channels: runs 8 (NR cq + r) .. + 8
  float qv[CQ];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[8 * r + i] = q[8 * (NR * cq + r) + i];
  // the K and V values of a block this lane needs
  struct Blk {
    float k[CQ];
    float4 v[NE][4];
  };
  bool bad = false;
  auto load = [&](int blk, Blk& x) {
    int phys = __builtin_amdgcn_readfirstlane(row[blk]);
    if (phys < 0 || phys >= a.num_blocks) {
      bad = true;
      phys = 0;
    }
    const float* kt = kc + int64_t(phys) * block_stride;
    const float* vt = vc + int64_t(phys) * block_stride;
#pragma unroll
    for (int r = 0; r < NR; ++r) {  // K (t, d) at (d / 8) 128 + 8 t + d % 8
      const float4* kp = reinterpret_cast<const float4*>(kt + (NR * cq + r) * 128 + tok * 8);
      const float4 k0 = kp[0], k1 = kp[1];
      x.k[8 * r + 0] = k0.x; x.k[8 * r + 1] = k0.y; x.k[8 * r + 2] = k0.z; x.k[8 * r + 3] = k0.w;
      x.k[8 * r + 4] = k1.x; x.k[8 * r + 5] = k1.y; x.k[8 * r + 6] = k1.z; x.k[8 * r + 7] = k1.w;
    }
#pragma unroll
    for (int e = 0; e < NE; ++e) {  // V (t, d) at (d / 32) 512 + (t / 4) 128 + v_elem's lane part
      const int d = lane + 64 * e;
      const float* vd = vt + v_elem(0, d);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) x.v[e][g4] = *reinterpret_cast<const float4*>(vd + 128 * g4);
    }
  };
  float acc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = 0.f;
  float m = -INFINITY, lsum = 0.f;
  Blk cur, nxt;
  load(blk0, cur);
  for (int blk = blk0; blk <= blk1; ++blk) {
    if (blk < blk1) load(blk + 1, nxt);
    float part_dot = 0.f;
#pragma unroll
    for (int i = 0; i < CQ; ++i) part_dot = fmaf(qv[i], cur.k[i], part_dot);
    part_dot += __shfl_xor(part_dot, 16);
    part_dot += __shfl_xor(part_dot, 32);
    const int tp = blk * kBlock + tok;
    const float sc = (tp >= t_lo && tp < t_hi) ? part_dot * a.scale_log2e : -INFINITY;
    float bmax = sc;
#pragma unroll
    for (int x = 1; x < 16; x <<= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, x));
    // every visited block holds a visible position, so the block max is finite
    const float mnew = fmaxf(m, bmax);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    const float p = __builtin_amdgcn_exp2f(sc - mnew);
    float psum = p;
#pragma unroll
    for (int x = 1; x < 16; x <<= 1) psum += __shfl_xor(psum, x);
    lsum = lsum * alpha + psum;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      float o = acc[e] * alpha;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        // invisible positions have weight 0, but their V slots may hold NaN
        const float4 v = cur.v[e][g4];
        const float w0 = __shfl(p, 4 * g4 + 0), w1 = __shfl(p, 4 * g4 + 1);
        const float w2 = __shfl(p, 4 * g4 + 2), w3 = __shfl(p, 4 * g4 + 3);
        const int t0 = blk * kBlock + 4 * g4;
        o = (t0 + 0 >= t_lo && t0 + 0 < t_hi) ? fmaf(w0, v.x, o) : o;
        o = (t0 + 1 >= t_lo && t0 + 1 < t_hi) ? fmaf(w1, v.y, o) : o;
        o = (t0 + 2 >= t_lo && t0 + 2 < t_hi) ? fmaf(w2, v.z, o) : o;
        o = (t0 + 3 >= t_lo && t0 + 3 < t_hi) ? fmaf(w3, v.w, o) : o;
      }
      acc[e] = o;
    }
    m = mnew;
    if (blk < blk1) cur = nxt;
  }
  if (nparts == 1) {
    const float inv = bad ? __builtin_nanf("") : 1.0f / lsum;
#pragma unroll
    for (int e = 0; e < NE; ++e) a.out[head * D + lane + 64 * e] = acc[e] * inv;
  } else {
    float* dst = a.ws_o + (head * a.max_parts + part) * D;
#pragma unroll
    for (int e = 0; e < NE; ++e) dst[lane + 64 * e] = acc[e];
    if (lane == 0) {
      a.ws_m[head * a.max_parts + part] = bad ? __builtin_nanf("") : m;
      a.ws_l[head * a.max_parts + part] = lsum;
    }
  }
}

template <int D>
__global__ __launch_bounds__(64) void lse_reduce_kernel(DecodeArgs a) {
  // one wavefront per (sequence, query head): lane l holds channels l + 64 k
  constexpr int NK = D / 64;
  const int lane = threadIdx.x;
  const int64_t head = blockIdx.x;
  const int b = static_cast<int>(head / a.num_q_heads);
  const int L = a.lens[b];
  if (!len_ok(L, a) || L == 0) return;
  const int base = first_block_of(a, L) * kBlock;
  const int nparts = (L - base + a.part_tokens - 1) / a.part_tokens;
  if (nparts <= 1) return;
  const float* mp = a.ws_m + head * a.max_parts;
  const float* lp = a.ws_l + head * a.max_parts;
  const float* op = a.ws_o + head * a.max_parts * D;
  // reference max and normaliser, partitions spread over the lanes
  float M = -INFINITY;
  bool bad = false;
  for (int p = lane; p < nparts; p += 64) {
    const float mv = mp[p];
    bad |= (mv != mv);
    M = fmaxf(M, mv);
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) M = fmaxf(M, __shfl_xor(M, s));
  bad = __builtin_amdgcn_ballot_w64(bad) != 0;
  float den = 0.f;
  for (int p = lane; p < nparts; p += 64) den = fmaf(__builtin_amdgcn_exp2f(mp[p] - M), lp[p], den);
  den = wave_sum(den);
  const float inv = bad ? __builtin_nanf("") : 1.0f / den;
  // out = sum_p 2^(m_p - M) o_p / den: partition p's factor is computed by
  // lane p % 64 and read from it; its D values are one coalesced load per k
  float acc[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k) acc[k] = 0.f;
  for (int p0 = 0; p0 < nparts; p0 += 64) {
    const int n = min(64, nparts - p0);
    const float w = lane < n ? __builtin_amdgcn_exp2f(mp[p0 + lane] - M) : 0.f;
    const float* o0 = op + int64_t(p0) * D + lane;
    auto fold = [&](int i) {
      const float wi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), i));
#pragma unroll
      for (int k = 0; k < NK; ++k) acc[k] = fmaf(wi, o0[int64_t(i) * D + 64 * k], acc[k]);
    };
    int i = 0;
    for (; i + 4 <= n; i += 4) {  // four partitions' loads in flight together
      fold(i);
      fold(i + 1);
      fold(i + 2);
      fold(i + 3);
    }
    for (; i < n; ++i) fold(i);
  }
#pragma unroll
  for (int k = 0; k < NK; ++k) a.out[head * D + 64 * k + lane] = acc[k] * inv;
}

// ------------------------------------------------------------------ measurement
// Streaming read: workgroup w (one wavefront) reads its own contiguous chunk
// with 1 KiB per load instruction and non-temporal 16-byte buffer loads
// (the same access form as the decode kernel), folding the data into one
// word per workgroup so the loads are not dead code.
__global__ __launch_bounds__(64) void stream_read_kernel(const char* __restrict__ src, int64_t bytes,
                                                         int64_t chunk, uint32_t* __restrict__ sink) {
  const int64_t begin = int64_t(blockIdx.x) * chunk;
  if (begin >= bytes) return;
  const int n = static_cast<int>(min(chunk, bytes - begin));
  const __amdgpu_buffer_rsrc_t r = tile_rsrc(src + begin, n);
  uint32_t acc = 0;
  for (int off = 0; off < n; off += 8 * 1024) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           r, off + u * 1024 + threadIdx.x * 16, 0, 2));
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;  // practically never taken
}

// ------------------------------------------------------------------ host helpers
bool debug_checks() {
  const char* v = std::getenv("PKV_DEBUG");
  return v && v[0] == '1';
}

// PKV_DEBUG check of a device slot mapping: in range and unique.  Synchronizes.
pkv_status check_slots(const int64_t* slot_mapping, int32_t num_tokens, int64_t num_slots,
                       hipStream_t stream) {
  std::vector<int64_t> host(num_tokens);
  if (hipStreamSynchronize(stream) != hipSuccess ||
      hipMemcpy(host.data(), slot_mapping, sizeof(int64_t) * num_tokens, hipMemcpyDeviceToHost) !=
          hipSuccess)
    return PKV_ERR_HIP;
  std::vector<char> seen(num_slots, 0);
  for (int64_t s : host) {
    if (s < 0) continue;
    if (s >= num_slots || seen[s]) return PKV_ERR_INVALID;
    seen[s] = 1;
  }
  return PKV_OK;
}


// Blocks kept in flight per wavefront by the bf16 decode kernel (2..4);
// PKV_DECODE_STAGES overrides the default for tuning.
int pipeline_stages() {
  static int st = [] {
    const char* v = std::getenv("PKV_DECODE_STAGES");
    int x = v ? std::atoi(v) : 0;
    return (x >= 2 && x <= 4) ? x : 3;
  }();
  return st;
}

// Cache policy of the bf16 decode K/V loads (0, 2 = non-temporal, 18);
// PKV_DECODE_CACHE overrides the default for tuning.
int decode_cache_policy() {
  static int aux = [] {
    const char* v = std::getenv("PKV_DECODE_CACHE");
    int x = v ? std::atoi(v) : 2;
    return (x == 0 || x == 2 || x == 18) ? x : 2;
  }();
  return aux;
}

// The balanced kernel also keeps the next segment's query fragments per
// stage, so it defaults to 2 stages (measured as fast as 3 on MI355X, with
// fewer registers); PKV_DECODE_STAGES=3 selects 3.
int pipeline_stages_balanced() {
  const char* v = std::getenv("PKV_DECODE_STAGES");
  return (v && std::atoi(v) == 3) ? 3 : 2;
}

int elem_size(pkv_dtype dt) { return dt == PKV_F32 ? 4 : (dt == PKV_BF16 ? 2 : 0); }

int resolve_partition(int32_t partition_size) {
  return partition_size == 0 ? kDefaultPartition : partition_size;
}

// Waves of the balanced decode grid: every wave slot of the current device
// (8 one-wave workgroups per compute unit at the kernel's register use);
// PKV_BALANCED_WAVES overrides it for tuning.  0 if the device query fails.
int balanced_waves() {
  const char* v = std::getenv("PKV_BALANCED_WAVES");
  if (v && std::atoi(v) > 0) return std::atoi(v);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cus * 8;
}

// Compute units of the current device (0 if the query fails).
int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cus;
}

// Balanced-mode scratch: per wave two partial states (D + 2 floats per head
// of the group), then the per-CU overflow slots of the per-CU form, then one
// 8-byte arrival counter per (sequence, kv head).
size_t balanced_states_bytes(int waves, int group, int head_dim) {
  return (size_t(waves) * 2 * group * (head_dim + 2) * sizeof(float) + 255) & ~size_t(255);
}
size_t cu_overflow_bytes(int cus, int over_slots, int group, int head_dim) {
  return (size_t(cus) * over_slots * cu_state_floats(group, head_dim) * sizeof(float) + 255) &
         ~size_t(255);
}
// Overflow slots per CU of the per-CU form: every slot beyond LDS (any mix
// of shares and chunks), or only those the fixed shares can need.
int cu_over_slots(int group, int head_dim, int num_seqs, bool static_only) {
  const int cap = cu_lds_slots(group, head_dim, num_seqs < kCuMaxSeqs ? num_seqs : kCuMaxSeqs);
  const int over = (static_only ? kCuStaticSlots : kCuSlots) - cap;
  return over > 0 ? over : 0;
}
size_t balanced_workspace_bytes(int waves, int group, int head_dim, int num_seqs,
                                int num_kv_heads) {
  return balanced_states_bytes(waves, group, head_dim) +
         cu_overflow_bytes(device_cus(), cu_over_slots(group, head_dim, num_seqs, false), group,
                           head_dim) +
         size_t(num_seqs) * num_kv_heads * 8;
}

// Scratch of the allocation-free decode entry point: one array per GPU,
// resident until the process ends.  Host code never passes `scratch`
// itself to a kernel (in host code the name is a host-side stand-in);
// scratch_device() resolves this GPU's copy once, with the device current.
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr int kScratchMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchMaxDevices] = {};

// Per-CU form parameters: each wavefront's fixed share of its CU's range
// (per mille) and the smallest chunk.  The default gives the whole range to
// fixed shares: on MI355X a CU finishes its range at the same time whether
// its wavefronts share it out dynamically or not (the CU's aggregate read
// rate is the limit, and wavefronts that finish early leave it to the
// others), and chunks only add partial states.  PKV_CU_STATIC_PERMILLE and
// PKV_CU_CHUNK_MIN override them for tuning and tests, PKV_DECODE_SPLIT=wave
// selects the per-wave form.
bool cu_split_enabled() {
  const char* v = std::getenv("PKV_DECODE_SPLIT");
  return !(v && std::strcmp(v, "wave") == 0);
}

// Launch tag for the arrival counters: a counter left by an earlier launch
// carries an older tag and is read as zero, so counters never need clearing.
unsigned next_epoch() {
  static unsigned e = 0x5EED0001u;
  e = e + 1 == 0 ? 1 : e + 1;
  return e;
}

int64_t max_parts_for(int32_t max_context_len, int part) {
  return max_context_len <= 0 ? 1 : (int64_t(max_context_len) + part - 1) / part;
}

struct Profiler {
  bool on = false;
  std::vector<hipEvent_t> pool;  // pairs: 2k = start, 2k+1 = stop
  size_t used = 0;
  int every = 1;      // time calls 0, every, 2 every, ... since begin
  int64_t calls = 0;  // decode calls since begin
};
Profiler g_prof;
constexpr size_t kMaxProfiled = 8192;

}  // namespace

template <int D, int ST>
void launch_decode_bf16_st(unsigned grid, hipStream_t stream, const DecodeArgs& a) {
  switch (decode_cache_policy()) {
    case 0: hipLaunchKernelGGL((decode_bf16_kernel<D, ST, 0>), grid, dim3(64), 0, stream, a); break;
    case 18: hipLaunchKernelGGL((decode_bf16_kernel<D, ST, 18>), grid, dim3(64), 0, stream, a); break;
    default: hipLaunchKernelGGL((decode_bf16_kernel<D, ST, 2>), grid, dim3(64), 0, stream, a); break;
  }
}

void launch_decode_bf16(unsigned grid, hipStream_t stream, const DecodeArgs& a, int head_dim) {
  const int st = pipeline_stages();
  if (head_dim == 64) {
    launch_decode_bf16_st<64, 4>(grid, stream, a);
  } else if (st == 2) {
    launch_decode_bf16_st<128, 2>(grid, stream, a);
  } else if (st == 4) {
    launch_decode_bf16_st<128, 4>(grid, stream, a);
  } else {
    launch_decode_bf16_st<128, 3>(grid, stream, a);
  }
}

void launch_decode_bf16_balanced(unsigned grid, hipStream_t stream, const DecodeArgs& a,
                                 int head_dim) {
  const int aux = decode_cache_policy();
  if (head_dim == 64) {
    hipLaunchKernelGGL((decode_bf16_balanced_kernel<64, 3, 2>), grid, dim3(64), 0, stream, a);
  } else if (aux == 0) {
    hipLaunchKernelGGL((decode_bf16_balanced_kernel<128, 3, 0>), grid, dim3(64), 0, stream, a);
  } else if (pipeline_stages_balanced() == 3) {
    hipLaunchKernelGGL((decode_bf16_balanced_kernel<128, 3, 2>), grid, dim3(64), 0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_bf16_balanced_kernel<128, 2, 2>), grid, dim3(64), 0, stream, a);
  }
}

template <bool WIN>
void launch_decode_bf16_cu_w(unsigned grid, hipStream_t stream, const DecodeArgs& a, int head_dim,
                             bool fp8) {
  const dim3 block(64 * kCuWaves);
  if (fp8) {
    if (head_dim == 64)
      hipLaunchKernelGGL((decode_bf16_cu_kernel<64, 3, 2, true, WIN>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((decode_bf16_cu_kernel<128, 2, 2, true, WIN>), grid, block, 0, stream, a);
  } else if (head_dim == 64) {
    hipLaunchKernelGGL((decode_bf16_cu_kernel<64, 3, 2, false, WIN>), grid, block, 0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_bf16_cu_kernel<128, 2, 2, false, WIN>), grid, block, 0, stream, a);
  }
}

// The fused decode step (bf16 cache): per-CU kernel with STEP = true.
template <bool WIN>
void launch_decode_step_w(unsigned grid, hipStream_t stream, const DecodeArgs& a, int head_dim) {
  const dim3 block(64 * kCuWaves);
  if (head_dim == 64)
    hipLaunchKernelGGL((decode_bf16_cu_kernel<64, 3, 2, false, WIN, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_bf16_cu_kernel<128, 2, 2, false, WIN, true>), grid, block, 0, stream, a);
}

void launch_decode_bf16_cu(unsigned grid, hipStream_t stream, const DecodeArgs& a, int head_dim,
                           bool fp8) {
  if (a.window > 0)
    launch_decode_bf16_cu_w<true>(grid, stream, a, head_dim, fp8);
  else
    launch_decode_bf16_cu_w<false>(grid, stream, a, head_dim, fp8);
}

// ============================================================================ C ABI

extern "C" {

pkv_status paged_block_table_update(int32_t* block_tables, int64_t table_elems,
                                    const int32_t* updates, int32_t num_updates,
                                    hipStream_t stream) {
  if (num_updates < 0 || table_elems < 0) return PKV_ERR_INVALID;
  if (num_updates == 0) return PKV_OK;
  if (!block_tables || !updates) return PKV_ERR_INVALID;
  const int threads = 256;
  const int grid = (num_updates + threads - 1) / threads;
  hipLaunchKernelGGL(table_update_kernel, dim3(grid), dim3(threads), 0, stream, block_tables,
                     table_elems, updates, num_updates);
  return launch_status();
}

pkv_status paged_kv_write(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                          void* k_cache, void* v_cache, int32_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, int32_t num_blocks, pkv_dtype dtype,
                          hipStream_t stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0)
    return PKV_ERR_INVALID;
  if (head_dim % 32 != 0) return PKV_ERR_UNSUPPORTED;
  if (elem_size(dtype) == 0) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PKV_ERR_INVALID;
  const int64_t num_slots = int64_t(num_blocks) * kBlock;
  if (debug_checks()) {
    pkv_status st = check_slots(slot_mapping, num_tokens, num_slots, stream);
    if (st != PKV_OK) return st;
  }
  const int64_t total = int64_t(num_tokens) * num_kv_heads * (head_dim / 8);
  const int threads = 256;
  const int64_t grid = (total + threads - 1) / threads;
  if (dtype == PKV_BF16) {
    hipLaunchKernelGGL(kv_write_kernel<uint16_t>, dim3(grid), dim3(threads), 0, stream,
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                       slot_mapping, static_cast<uint16_t*>(k_cache),
                       static_cast<uint16_t*>(v_cache), total, num_kv_heads, head_dim, num_slots);
  } else {
    hipLaunchKernelGGL(kv_write_kernel<float>, dim3(grid), dim3(threads), 0, stream,
                       static_cast<const float*>(k_new), static_cast<const float*>(v_new),
                       slot_mapping, static_cast<float*>(k_cache), static_cast<float*>(v_cache),
                       total, num_kv_heads, head_dim, num_slots);
  }
  return launch_status();
}

pkv_status paged_kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                           void* k_cache, void* v_cache, int32_t num_tokens, int32_t num_kv_heads,
                           int32_t head_dim, int32_t num_blocks, pkv_dtype dtype,
                           int32_t* block_tables, int64_t table_elems, const int32_t* updates,
                           int32_t num_updates, hipStream_t stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0 ||
      num_updates < 0 || table_elems < 0)
    return PKV_ERR_INVALID;
  if (head_dim % 32 != 0 || elem_size(dtype) == 0) return PKV_ERR_UNSUPPORTED;
  if (num_tokens > 0 && (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache))
    return PKV_ERR_INVALID;
  if (num_updates > 0 && (!block_tables || !updates)) return PKV_ERR_INVALID;
  if (num_tokens == 0 && num_updates == 0) return PKV_OK;
  const int64_t num_slots = int64_t(num_blocks) * kBlock;
  if (debug_checks() && num_tokens > 0) {
    pkv_status st = check_slots(slot_mapping, num_tokens, num_slots, stream);
    if (st != PKV_OK) return st;
  }
  const int threads = 256;
  const int table_wgs = (num_updates + threads - 1) / threads;
  const int64_t total = int64_t(num_tokens) * num_kv_heads * (head_dim / 8);
  const int64_t grid = table_wgs + (total + threads - 1) / threads;
  if (dtype == PKV_BF16) {
    hipLaunchKernelGGL(append_kernel<uint16_t>, dim3(grid), dim3(threads), 0, stream,
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                       slot_mapping, static_cast<uint16_t*>(k_cache),
                       static_cast<uint16_t*>(v_cache), total, num_kv_heads, head_dim, num_slots,
                       block_tables, table_elems, updates, num_updates, table_wgs);
  } else {
    hipLaunchKernelGGL(append_kernel<float>, dim3(grid), dim3(threads), 0, stream,
                       static_cast<const float*>(k_new), static_cast<const float*>(v_new),
                       slot_mapping, static_cast<float*>(k_cache), static_cast<float*>(v_cache),
                       total, num_kv_heads, head_dim, num_slots, block_tables, table_elems,
                       updates, num_updates, table_wgs);
  }
  return launch_status();
}

pkv_status paged_kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs,
                                int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                                int32_t num_blocks, pkv_dtype dtype, hipStream_t stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0)
    return PKV_ERR_INVALID;
  const int esize = dtype == PKV_FP8_E4M3 ? 1 : elem_size(dtype);
  if (head_dim % 32 != 0 || esize == 0) return PKV_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !pairs) return PKV_ERR_INVALID;
  const int64_t run_bytes = int64_t(num_kv_heads) * kBlock * head_dim * esize;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, 2), dim3(256), 0, stream,
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), pairs,
                     run_bytes / 16, num_blocks);
  return launch_status();
}

pkv_status paged_kv_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                                const int32_t* pairs, int32_t num_pairs, int32_t num_kv_heads,
                                int32_t head_dim, int32_t src_num_blocks, int32_t dst_num_blocks,
                                pkv_dtype dtype, hipStream_t stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || src_num_blocks <= 0 ||
      dst_num_blocks <= 0)
    return PKV_ERR_INVALID;
  const int esize = dtype == PKV_FP8_E4M3 ? 1 : elem_size(dtype);
  if (head_dim % 32 != 0 || esize == 0) return PKV_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PKV_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !pairs) return PKV_ERR_INVALID;
  if (src_k == dst_k || src_v == dst_v) return PKV_ERR_INVALID;  // in-cache copies: copy_blocks
  const int64_t run_bytes = int64_t(num_kv_heads) * kBlock * head_dim * esize;
  hipLaunchKernelGGL(swap_blocks_kernel, dim3(num_pairs, 2), dim3(256), 0, stream,
                     static_cast<const uint4*>(src_k), static_cast<const uint4*>(src_v),
                     static_cast<uint4*>(dst_k), static_cast<uint4*>(dst_v), pairs, run_bytes / 16,
                     src_num_blocks, dst_num_blocks);
  return launch_status();
}

size_t paged_attention_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      partition_size < 0 || num_q_heads % num_kv_heads != 0)
    return 0;
  const int part = resolve_partition(partition_size);
  const int64_t mp = max_parts_for(max_context_len, part);
  size_t fixed = mp <= 1 ? 0 : size_t(num_seqs) * num_q_heads * mp * (head_dim + 2) * sizeof(float);
  if (partition_size != 0) return fixed;
  // partition_size 0: the balanced bf16 form (group of at most 16 heads)
  // or 512-token partitions for fp32 -- room for either
  const int group = num_q_heads / num_kv_heads;
  const size_t bal = balanced_workspace_bytes(balanced_waves(), group < 16 ? group : 16, head_dim,
                                              num_seqs, num_kv_heads);
  return fixed > bal ? fixed : bal;
}

}  // extern "C"

namespace {
// This GPU's copy of `scratch`, resolved once per device with the device
// current (nullptr if that fails).
void* scratch_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// Decode for every cache dtype; fp8 (E4M3 codes with tensor scales) runs
// only in the per-CU balanced form.  fixed_scratch: the allocation-free
// form -- per-CU split with fixed shares only, its partial states and
// arrival counters in this GPU's `scratch` (workspace arguments ignored).
pkv_status decode_impl(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                       float scale, int32_t window, int32_t partition_size, void* workspace,
                       size_t workspace_bytes, pkv_dtype kv_dtype, float k_scale, float v_scale,
                       float* out, hipStream_t stream, bool fixed_scratch = false,
                       const DecodeArgs* step = nullptr) {
  const bool fp8 = kv_dtype == PKV_FP8_E4M3;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_blocks <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0 || partition_size < 0 ||
      window < 0)
    return PKV_ERR_INVALID;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_INVALID;
  if (partition_size % 32 != 0) return PKV_ERR_INVALID;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (elem_size(kv_dtype) == 0 && !fp8) return PKV_ERR_UNSUPPORTED;
  if (fp8 && (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) ||
              !std::isfinite(v_scale)))
    return PKV_ERR_INVALID;
  if (fp8 && partition_size != 0) return PKV_ERR_UNSUPPORTED;
  if (step && (kv_dtype != PKV_BF16 || partition_size != 0)) return PKV_ERR_UNSUPPORTED;
  if (fixed_scratch && (kv_dtype == PKV_F32 || partition_size != 0)) return PKV_ERR_UNSUPPORTED;
  const int group = num_q_heads / num_kv_heads;
  if ((kv_dtype == PKV_BF16 || fp8) && group > 16) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return PKV_ERR_INVALID;
  const int part = resolve_partition(partition_size);
  const int64_t max_parts = max_parts_for(max_context_len, part);
  // one workgroup per (partition, sequence, head) must fit a 1D grid
  if (max_parts * num_seqs * num_q_heads > 0x7FFFFFFF) return PKV_ERR_UNSUPPORTED;
  const bool balanced = (kv_dtype == PKV_BF16 || fp8) && partition_size == 0;
  const int cus = balanced ? device_cus() : 0;
  // per-CU form: sequences whose tile-count prefix fits LDS, a tile list
  // indexed in 32 bits, and global partial-state slots (2 per CU) within
  // those of the per-wave grid
  const bool cu_shape = num_seqs <= kCuMaxSeqs &&
                        int64_t(num_seqs) * max_blocks_per_seq * num_kv_heads <
                            (int64_t(1) << 31) &&
                        cus > 0;
  DecodeArgs a{};
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.out = out;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.max_ctx = max_context_len;
  a.part_tokens = part;
  a.max_parts = static_cast<int>(max_parts);
  a.scale_log2e = scale * (fp8 ? k_scale : 1.0f) * 1.4426950408889634f;
  a.out_scale = fp8 ? v_scale : 1.0f;
  a.window = window;
  bool cu_form;
  int waves = 0;
  if (fixed_scratch) {
    if (!cu_shape) return PKV_ERR_UNSUPPORTED;
    // [2 cus][g][D] o, [2 cus][g] m, [2 cus][g] l | overflow | counters
    const size_t states = balanced_states_bytes(cus, group, head_dim);
    const int over = cu_over_slots(group, head_dim, num_seqs, true);
    const size_t overflow = cu_overflow_bytes(cus, over, group, head_dim);
    const size_t need = states + overflow + size_t(num_seqs) * num_kv_heads * 8;
    if (need > kScratchBytes) return PKV_ERR_UNSUPPORTED;
    char* base = static_cast<char*>(scratch_device());
    if (!base) return PKV_ERR_HIP;
    float* ws = reinterpret_cast<float*>(base);
    a.ws_o = a.ws_m = a.ws_l = nullptr;
    a.bw_o = ws;
    a.bw_m = ws + size_t(cus) * 2 * group * head_dim;
    a.bw_l = a.bw_m + size_t(cus) * 2 * group;
    a.cu_over = reinterpret_cast<float*>(base + states);
    a.over_slots = over;
    a.bw_count = reinterpret_cast<unsigned long long*>(base + states + overflow);
    a.static_permille = 1000;
    a.chunk_min = kCuStaticChunkMin;
    a.grid_waves = cus;
    cu_form = true;
  } else {
    waves = balanced ? balanced_waves() : 0;
    if (balanced && waves <= 0) return PKV_ERR_HIP;
    const size_t need =
        balanced ? balanced_workspace_bytes(waves, group, head_dim, num_seqs, num_kv_heads)
                 : paged_attention_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                  max_context_len,
                                                  partition_size == 0 ? kDefaultPartition
                                                                      : partition_size);
    if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_ERR_INVALID;
    const int64_t heads = int64_t(num_seqs) * num_q_heads;
    float* ws = static_cast<float*>(workspace);
    a.ws_o = ws;
    a.ws_m = ws ? ws + heads * max_parts * head_dim : nullptr;
    a.ws_l = ws ? a.ws_m + heads * max_parts : nullptr;
    a.grid_waves = waves;
    a.bw_o = balanced ? ws : nullptr;
    a.bw_m = balanced ? ws + size_t(waves) * 2 * group * head_dim : nullptr;
    a.bw_l = balanced ? a.bw_m + size_t(waves) * 2 * group : nullptr;
    const int over = cu_over_slots(group, head_dim, num_seqs, false);
    a.over_slots = over;
    a.cu_over = balanced ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                    balanced_states_bytes(waves, group, head_dim))
                         : nullptr;
    a.bw_count = balanced ? reinterpret_cast<unsigned long long*>(
                                static_cast<char*>(workspace) +
                                balanced_states_bytes(waves, group, head_dim) +
                                cu_overflow_bytes(cus, over, group, head_dim))
                          : nullptr;
    a.static_permille = env_int("PKV_CU_STATIC_PERMILLE", 1000, 0, 1000);
    a.chunk_min = env_int("PKV_CU_CHUNK_MIN", 4, 1, 1 << 20);
    cu_form = balanced && cu_split_enabled() && cu_shape && cus <= waves;
  }
  a.epoch = balanced ? next_epoch() : 0;
  if (fp8 && !cu_form) return PKV_ERR_UNSUPPORTED;
  if (step) {
    if (!cu_form) return PKV_ERR_UNSUPPORTED;
    a.k_new = step->k_new;
    a.v_new = step->v_new;
    a.slots = step->slots;
    a.tables_w = step->tables_w;
    a.table_elems = step->table_elems;
    a.upd = step->upd;
    a.n_upd = step->n_upd;
    a.lens_out = step->lens_out;
  }

  const bool prof = g_prof.on && g_prof.calls++ % g_prof.every == 0 &&
                    g_prof.used + 2 <= g_prof.pool.size();
  if (prof) (void)hipEventRecord(g_prof.pool[g_prof.used], stream);
  if (balanced) {
    if (step && a.window > 0)
      launch_decode_step_w<true>(static_cast<unsigned>(cus), stream, a, head_dim);
    else if (step)
      launch_decode_step_w<false>(static_cast<unsigned>(cus), stream, a, head_dim);
    else if (cu_form)
      launch_decode_bf16_cu(static_cast<unsigned>(cus), stream, a, head_dim, fp8);
    else
      launch_decode_bf16_balanced(static_cast<unsigned>(waves), stream, a, head_dim);
    if (prof) {
      (void)hipEventRecord(g_prof.pool[g_prof.used + 1], stream);
      g_prof.used += 2;
    }
    return launch_status();
  }
  if (kv_dtype == PKV_BF16) {
    const unsigned grid = static_cast<unsigned>(max_parts * num_seqs * num_kv_heads);
    launch_decode_bf16(grid, stream, a, head_dim);
  } else {
    const unsigned grid = static_cast<unsigned>(max_parts * num_seqs * num_q_heads);
    if (head_dim == 128)
      hipLaunchKernelGGL(decode_f32_kernel<128>, grid, dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL(decode_f32_kernel<64>, grid, dim3(64), 0, stream, a);
  }
  pkv_status st = launch_status();
  if (st == PKV_OK && max_parts > 1) {
    const unsigned rgrid = static_cast<unsigned>(int64_t(num_seqs) * num_q_heads);
    if (head_dim == 128)
      hipLaunchKernelGGL(lse_reduce_kernel<128>, dim3(rgrid), dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL(lse_reduce_kernel<64>, dim3(rgrid), dim3(64), 0, stream, a);
    st = launch_status();
  }
  // the timed span of a fixed-partition call covers its reduce as well
  if (prof) {
    (void)hipEventRecord(g_prof.pool[g_prof.used + 1], stream);
    g_prof.used += 2;
  }
  return st;
}
}  // namespace

extern "C" {

pkv_status paged_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t num_blocks,
                                  int32_t max_blocks_per_seq, int32_t max_context_len,
                                  float scale, int32_t partition_size, void* workspace,
                                  size_t workspace_bytes, pkv_dtype kv_dtype, float* out,
                                  hipStream_t stream) {
  if (kv_dtype == PKV_FP8_E4M3) return PKV_ERR_UNSUPPORTED;  // needs the scales
  return decode_impl(q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, num_blocks, max_blocks_per_seq, max_context_len,
                     scale, 0, partition_size, workspace, workspace_bytes, kv_dtype, 1.0f, 1.0f,
                     out, stream);
}

pkv_status paged_attention_decode_window(const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* block_tables, const int32_t* context_lens,
                                         int32_t num_seqs, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                         int32_t max_blocks_per_seq, int32_t max_context_len,
                                         float scale, int32_t window, int32_t partition_size,
                                         void* workspace, size_t workspace_bytes,
                                         pkv_dtype kv_dtype, float k_scale, float v_scale,
                                         float* out, hipStream_t stream) {
  if (kv_dtype != PKV_FP8_E4M3) k_scale = v_scale = 1.0f;
  return decode_impl(q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, num_blocks, max_blocks_per_seq, max_context_len,
                     scale, window, partition_size, workspace, workspace_bytes, kv_dtype, k_scale,
                     v_scale, out, stream);
}

pkv_status paged_kv_append_decode(const void* q, const void* k_new, const void* v_new,
                                  const int64_t* slot_mapping, void* k_cache, void* v_cache,
                                  int32_t* block_tables, const int32_t* context_lens_in,
                                  int32_t* context_lens_out, const int32_t* updates,
                                  int32_t num_updates, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                  int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                                  int32_t window, void* workspace, size_t workspace_bytes,
                                  pkv_dtype kv_dtype, float* out, hipStream_t stream) {
  if (num_updates < 0 || num_seqs < 0) return PKV_ERR_INVALID;
  if (num_seqs > 0 && (!k_new || !v_new || !slot_mapping || !context_lens_out ||
                       context_lens_out == context_lens_in))
    return PKV_ERR_INVALID;
  if (num_updates > 0 && !updates) return PKV_ERR_INVALID;
  DecodeArgs st{};
  st.k_new = k_new;
  st.v_new = v_new;
  st.slots = slot_mapping;
  st.tables_w = block_tables;
  st.table_elems = int64_t(num_seqs) * max_blocks_per_seq;
  st.upd = updates;
  st.n_upd = num_updates;
  st.lens_out = context_lens_out;
  return decode_impl(q, k_cache, v_cache, block_tables, context_lens_in, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, num_blocks, max_blocks_per_seq, max_context_len,
                     scale, window, 0, workspace, workspace_bytes, kv_dtype, 1.0f, 1.0f, out,
                     stream, false, &st);
}

pkv_status paged_attention_decode_noalloc(const void* q, const void* k_cache,
                                          const void* v_cache, const int32_t* block_tables,
                                          const int32_t* context_lens, int32_t num_seqs,
                                          int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t num_blocks,
                                          int32_t max_blocks_per_seq, int32_t max_context_len,
                                          float scale, int32_t window, pkv_dtype kv_dtype,
                                          float k_scale, float v_scale, float* out,
                                          hipStream_t stream) {
  if (kv_dtype != PKV_FP8_E4M3) k_scale = v_scale = 1.0f;
  return decode_impl(q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, num_blocks, max_blocks_per_seq, max_context_len,
                     scale, window, 0, nullptr, 0, kv_dtype, k_scale, v_scale, out, stream,
                     true);
}

pkv_status paged_attention_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t num_blocks,
                                      int32_t max_blocks_per_seq, int32_t max_context_len,
                                      float scale, float k_scale, float v_scale, void* workspace,
                                      size_t workspace_bytes, float* out, hipStream_t stream) {
  return decode_impl(q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, num_blocks, max_blocks_per_seq, max_context_len,
                     scale, 0, 0, workspace, workspace_bytes, PKV_FP8_E4M3, k_scale, v_scale,
                     out, stream);
}

pkv_status paged_kv_write_fp8(const void* k_new, const void* v_new, pkv_dtype src_dtype,
                              const int64_t* slot_mapping, void* k_cache, void* v_cache,
                              int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                              int32_t num_blocks, float k_scale, float v_scale,
                              hipStream_t stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0)
    return PKV_ERR_INVALID;
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return PKV_ERR_INVALID;
  if (head_dim % 32 != 0) return PKV_ERR_UNSUPPORTED;
  if (src_dtype != PKV_BF16 && src_dtype != PKV_F32) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PKV_ERR_INVALID;
  const int64_t num_slots = int64_t(num_blocks) * kBlock;
  if (debug_checks()) {
    pkv_status st = check_slots(slot_mapping, num_tokens, num_slots, stream);
    if (st != PKV_OK) return st;
  }
  const float k_inv = 1.0f / k_scale, v_inv = 1.0f / v_scale;
  const int64_t total = int64_t(num_tokens) * num_kv_heads * (head_dim / 8);
  const int threads = 256;
  const int64_t grid = (total + threads - 1) / threads;
  if (src_dtype == PKV_BF16)
    hipLaunchKernelGGL(kv_write_fp8_kernel<uint16_t>, dim3(grid), dim3(threads), 0, stream,
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                       slot_mapping, static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache),
                       total, num_kv_heads, head_dim, num_slots, k_inv, v_inv);
  else
    hipLaunchKernelGGL(kv_write_fp8_kernel<float>, dim3(grid), dim3(threads), 0, stream,
                       static_cast<const float*>(k_new), static_cast<const float*>(v_new),
                       slot_mapping, static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache),
                       total, num_kv_heads, head_dim, num_slots, k_inv, v_inv);
  return launch_status();
}

pkv_status pkv_stream_read(const void* buf, size_t bytes, void* sink, hipStream_t stream) {
  if (!buf || !sink || bytes < 16) return PKV_ERR_INVALID;
  constexpr int kGrid = 8192;
  const int64_t total = static_cast<int64_t>(bytes & ~size_t(15));
  // per-workgroup chunks of whole KiB, each below 2 GiB
  const int64_t chunk = ((total + kGrid - 1) / kGrid + 1023) & ~int64_t(1023);
  if (chunk >= (int64_t(1) << 31)) return PKV_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(stream_read_kernel, dim3(kGrid), dim3(64), 0, stream,
                     static_cast<const char*>(buf), total, chunk, static_cast<uint32_t*>(sink));
  return launch_status();
}

pkv_status pkv_profile_begin(int32_t every) {
  if (every < 1) return PKV_ERR_INVALID;
  if (g_prof.pool.empty()) {
    g_prof.pool.resize(2 * kMaxProfiled);
    // timing only: no system-scope fence when an event is reached, so a
    // recorded pair costs the stream little more than its two markers
    for (auto& e : g_prof.pool)
      if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
        g_prof.pool.clear();
        return PKV_ERR_HIP;
      }
  }
  g_prof.used = 0;
  g_prof.calls = 0;
  g_prof.every = every;
  g_prof.on = true;
  return PKV_OK;
}

pkv_status pkv_profile_durations(float* out_ms, int32_t capacity, int32_t* num_launches) {
  if (!num_launches || capacity < 0 || (capacity > 0 && !out_ms)) return PKV_ERR_INVALID;
  int32_t k = 0;
  for (size_t i = 0; i + 1 < g_prof.used; i += 2, ++k) {
    float ms = 0.f;
    if (hipEventSynchronize(g_prof.pool[i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, g_prof.pool[i], g_prof.pool[i + 1]) != hipSuccess)
      return PKV_ERR_HIP;
    if (k < capacity) out_ms[k] = ms;
  }
  *num_launches = k;
  return PKV_OK;
}

pkv_status pkv_profile_end(int32_t* num_launches, double* total_ms) {
  if (!num_launches || !total_ms) return PKV_ERR_INVALID;
  g_prof.on = false;
  double total = 0.0;
  for (size_t i = 0; i + 1 < g_prof.used; i += 2) {
    float ms = 0.f;
    if (hipEventSynchronize(g_prof.pool[i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, g_prof.pool[i], g_prof.pool[i + 1]) != hipSuccess)
      return PKV_ERR_HIP;
    total += ms;
  }
  *num_launches = static_cast<int32_t>(g_prof.used / 2);
  *total_ms = total;
  g_prof.used = 0;
  return PKV_OK;
}

}  // extern "C"
