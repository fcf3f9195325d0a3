// Device side of libpagedkv: HIP kernels for gfx950 (CDNA4) and the C ABI
// entry points that launch them.
//
// Kernels:
//   table_update   block-table deltas into the device-resident tables
//   kv_write       scatter of new tokens' K/V through the slot mapping
//   copy_blocks    whole-block copies for copy-on-write
//   decode_bf16    PagedAttention decode, bf16 cache, matrix cores
//   decode_f32     PagedAttention decode, fp32 cache, vector ALU
//   lse_reduce     log-sum-exp merge of partitions
//
// Sources: "PagedAttention por dentro" (blog.lo0.es), sections "La tabla de
// paginas (block table)", "Copy-on-write para sampling paralelo" and "El
// kernel CUDA" (attention walks the context in block-aligned chunks, each
// located through the table); "Como funciona realmente vLLM"
// (alexanderzelada.com), "Que es el mecanismo de atencion" and
// "PagedAttention: ..." (scattered blocks are read in place through the
// table, never gathered into a contiguous buffer).
//
// Decode design (bf16).  One wavefront (64 lanes) owns one
// (sequence, kv head, partition) work item and walks that partition's
// blocks through the block table.  The cache tile order (pagedkv.h) makes
// lane l's 16-byte piece j of a tile exactly its matrix-core operand:
//   K piece j = 8 channels 32j + 8(l/16) .. +8 of token l%16
//       -> A operand of v_mfma_f32_16x16x32_bf16 (rows = tokens, k = channels)
//   V piece j = 4 tokens 4(l/16) .. +4 at channel 32j + l%16 (low half) and
//       channel 32j + 16 + l%16 (high half)
//       -> B operands of v_mfma_f32_16x16x16_bf16 (k = tokens, cols = channels)
// so each load instruction of the wave reads 1 KiB of contiguous memory and
// nothing passes through LDS or gets reshuffled.  Scores come out as
// S^T[token 4(l/16)+i][query head l%16] -- exactly the A-operand layout of
// the P.V product (rows = heads, k = tokens) -- so up to 16 query heads of a
// kv head share one pass over the tile.  Softmax weights are split into a
// bf16 high part and a bf16 residual so that P.V keeps ~16 bits of weight
// precision; accumulation is fp32 throughout.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "pagedkv.h"

namespace {

constexpr int kBlock = PKV_BLOCK_SIZE;
constexpr int kDefaultPartition = 512;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ in-tile order
__host__ __device__ inline int k_elem(int t, int d) { return (d >> 3) * 128 + t * 8 + (d & 7); }
__host__ __device__ inline int v_elem(int t, int d) {
  return (d >> 5) * 512 + (t >> 2) * 128 + (d & 15) * 8 + ((d >> 4) & 1) * 4 + (t & 3);
}

// ------------------------------------------------------------------ wave helpers
__device__ inline float group_max(float x) {  // over lanes l, l^16, l^32, l^48
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ inline float group_sum(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}
__device__ inline float wave_sum(float x) {
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

__device__ inline uint32_t bf16_bits_rne(float f) {
  // round to nearest even; inputs here are finite and non-negative weights
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ------------------------------------------------------------------ A2: table deltas
__global__ void table_update_kernel(int32_t* __restrict__ tables, int64_t elems,
                                    const int32_t* __restrict__ upd, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  int64_t idx = upd[2 * i];
  if (idx >= 0 && idx < elems) tables[idx] = upd[2 * i + 1];
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
  const int64_t slot = slots[i];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot >> 4;
  const int t = static_cast<int>(slot & 15);
  const int64_t src = (i * num_kv_heads + h) * head_dim + c * 8;
  const int64_t tile = (blk * num_kv_heads + h) * int64_t(kBlock) * head_dim;
  T kv[8], vv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    kv[e] = k_new[src + e];
    vv[e] = v_new[src + e];
  }
  // K: the 8 channels of a group are contiguous for a token
#pragma unroll
  for (int e = 0; e < 8; ++e) kc[tile + k_elem(t, c * 8 + e)] = kv[e];
#pragma unroll
  for (int e = 0; e < 8; ++e) vc[tile + v_elem(t, c * 8 + e)] = vv[e];
}

// ------------------------------------------------------------------ A4: block copies
// blockIdx.x = pair, blockIdx.y = 0 (K) / 1 (V); a block of all heads is one
// contiguous run of `run16` 16-byte words.
__global__ void copy_blocks_kernel(uint4* __restrict__ kc, uint4* __restrict__ vc,
                                   const int32_t* __restrict__ pairs, int64_t run16,
                                   int num_blocks) {
  const int32_t src = pairs[2 * blockIdx.x];
  const int32_t dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  uint4* base = blockIdx.y ? vc : kc;
  const uint4* s = base + int64_t(src) * run16;
  uint4* d = base + int64_t(dst) * run16;
  for (int64_t i = threadIdx.x; i < run16; i += blockDim.x) d[i] = s[i];
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
  int num_q_heads, num_kv_heads, group;
  int num_blocks, max_blocks, max_ctx, part_tokens, max_parts;
  float scale_log2e;
};

// Length check shared by the kernels: a bad length poisons the sequence.
__device__ inline bool len_ok(int L, const DecodeArgs& a) {
  return L >= 0 && L <= a.max_ctx && int64_t(L) <= int64_t(a.max_blocks) * kBlock;
}

template <int D>
__global__ __launch_bounds__(64) void decode_bf16_kernel(DecodeArgs a) {
  constexpr int NJ = D / 32;  // 16-byte pieces per lane per tile (K and V each)
  constexpr int NT = D / 16;  // 16-channel output tiles
  constexpr int64_t TILE = int64_t(kBlock) * D;

  const int lane = threadIdx.x;
  const int part = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
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
  const int nparts = (L + a.part_tokens - 1) / a.part_tokens;
  if (part >= nparts) return;
  const int t_begin = part * a.part_tokens;
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

  const uint16_t* kbase = static_cast<const uint16_t*>(a.kc) + kvh * TILE + lane * 8;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.vc) + kvh * TILE + lane * 8;
  const int64_t block_stride = int64_t(a.num_kv_heads) * TILE;

  f32x4 o[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;  // running max of this lane's head (log2 domain)
  float lsum = 0.f;     // this lane's share of the sum of weights
  bool bad = false;

  auto load_block = [&](int i, uint4 (&kr)[NJ], uint4 (&vr)[NJ]) {
    int phys = __builtin_amdgcn_readfirstlane(row[i]);
    if (phys < 0 || phys >= a.num_blocks) {
      bad = true;
      phys = 0;
    }
    const int64_t off = int64_t(phys) * block_stride;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      kr[j] = *reinterpret_cast<const uint4*>(kbase + off + 512 * j);
      vr[j] = *reinterpret_cast<const uint4*>(vbase + off + 512 * j);
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
    for (int r = 0; r < 4; ++r) sv[r] = (tb + r < t_end) ? s[r] * a.scale_log2e : -INFINITY;
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
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      hi[r] = bf16_bits_rne(p[r]);
      lo[r] = bf16_bits_rne(p[r] - __uint_as_float(hi[r] << 16));
    }
    const s16x4 phi = __builtin_bit_cast(s16x4, make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)));
    const s16x4 plo = __builtin_bit_cast(s16x4, make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)));
    if (t_begin + i * kBlock + kBlock > t_end) {
      // partial block: zero V of slots past the context (they may hold NaN)
      const uint32_t m01 = (tb + 0 < t_end ? 0x0000FFFFu : 0u) | (tb + 1 < t_end ? 0xFFFF0000u : 0u);
      const uint32_t m23 = (tb + 2 < t_end ? 0x0000FFFFu : 0u) | (tb + 3 < t_end ? 0xFFFF0000u : 0u);
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

  // two-stage pipeline: the next block's loads are in flight while one computes
  uint4 ka[NJ], va[NJ], kb[NJ], vb[NJ];
  load_block(0, ka, va);
  if (nblk > 1) load_block(1, kb, vb);
  for (int i = 0; i < nblk; i += 2) {
    compute_block(i, ka, va);
    if (i + 2 < nblk) load_block(i + 2, ka, va);
    if (i + 1 < nblk) {
      compute_block(i + 1, kb, vb);
      if (i + 3 < nblk) load_block(i + 3, kb, vb);
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

// ------------------------------------------------------------------ A5: decode, fp32
// One wave per (sequence, query head, partition); lane holds channels lane
// and lane + 64.  Plain vector-ALU form for the fp32 cache.
template <int D>
__global__ __launch_bounds__(64) void decode_f32_kernel(DecodeArgs a) {
  constexpr int NE = D / 64;
  constexpr int64_t TILE = int64_t(kBlock) * D;
  const int lane = threadIdx.x;
  const int part = blockIdx.x;
  const int hq = blockIdx.y;
  const int b = blockIdx.z;
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
  const int nparts = (L + a.part_tokens - 1) / a.part_tokens;
  if (part >= nparts) return;
  const int t_begin = part * a.part_tokens;
  const int t_end = min(L, t_begin + a.part_tokens);
  const int32_t* row = a.tables + int64_t(b) * a.max_blocks;
  const float* q = static_cast<const float*>(a.q) + head * D;
  const float* kc = static_cast<const float*>(a.kc) + kvh * TILE;
  const float* vc = static_cast<const float*>(a.vc) + kvh * TILE;
  const int64_t block_stride = int64_t(a.num_kv_heads) * TILE;
  float qv[NE], acc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    qv[e] = q[lane + 64 * e];
    acc[e] = 0.f;
  }
  float m = -INFINITY, lsum = 0.f;
  bool bad = false;
  for (int t = t_begin; t < t_end; ++t) {
    int phys = __builtin_amdgcn_readfirstlane(row[t / kBlock]);
    if (phys < 0 || phys >= a.num_blocks) {
      bad = true;
      phys = 0;
    }
    const float* kt = kc + int64_t(phys) * block_stride;
    const float* vt = vc + int64_t(phys) * block_stride;
    const int slot = t % kBlock;
    float part_dot = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) part_dot = fmaf(qv[e], kt[k_elem(slot, lane + 64 * e)], part_dot);
    const float s = wave_sum(part_dot) * a.scale_log2e;
    const float mnew = fmaxf(m, s);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    const float p = __builtin_amdgcn_exp2f(s - mnew);
    lsum = lsum * alpha + p;
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = fmaf(p, vt[v_elem(slot, lane + 64 * e)], acc[e] * alpha);
    m = mnew;
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

// ------------------------------------------------------------------ A6: LSE reduce
// One wave per (sequence, query head) with more than one partition:
//   M = max_p m_p,  l = sum_p l_p 2^(m_p - M),  out = sum_p o_p 2^(m_p - M) / l
template <int D>
__global__ __launch_bounds__(64) void lse_reduce_kernel(DecodeArgs a) {
  constexpr int NE = D / 64;
  const int lane = threadIdx.x;
  const int64_t head = blockIdx.x;  // b * Hq + hq
  const int b = static_cast<int>(head / a.num_q_heads);
  const int L = a.lens[b];
  if (!len_ok(L, a) || L == 0) return;
  const int nparts = (L + a.part_tokens - 1) / a.part_tokens;
  if (nparts <= 1) return;
  const float* mp = a.ws_m + head * a.max_parts;
  const float* lp = a.ws_l + head * a.max_parts;
  const float* op = a.ws_o + head * a.max_parts * D;
  float M = -INFINITY;
  bool bad = false;
  for (int p = 0; p < nparts; ++p) {
    const float mv = mp[p];
    bad |= (mv != mv);
    M = fmaxf(M, mv);
  }
  float acc[NE], den = 0.f;
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float w = __builtin_amdgcn_exp2f(mp[p] - M);
    den = fmaf(w, lp[p], den);
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = fmaf(w, op[int64_t(p) * D + lane + 64 * e], acc[e]);
  }
  const float inv = bad ? __builtin_nanf("") : 1.0f / den;
#pragma unroll
  for (int e = 0; e < NE; ++e) a.out[head * D + lane + 64 * e] = acc[e] * inv;
}

// ------------------------------------------------------------------ host helpers
bool debug_checks() {
  const char* v = std::getenv("PKV_DEBUG");
  return v && v[0] == '1';
}

pkv_status launch_status() {
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int elem_size(pkv_dtype dt) { return dt == PKV_F32 ? 4 : (dt == PKV_BF16 ? 2 : 0); }

int resolve_partition(int32_t partition_size) {
  return partition_size == 0 ? kDefaultPartition : partition_size;
}

int64_t max_parts_for(int32_t max_context_len, int part) {
  return max_context_len <= 0 ? 1 : (int64_t(max_context_len) + part - 1) / part;
}

struct Profiler {
  bool on = false;
  std::vector<hipEvent_t> pool;  // pairs: 2k = start, 2k+1 = stop
  size_t used = 0;
};
Profiler g_prof;
constexpr size_t kMaxProfiled = 8192;

}  // namespace

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
    std::vector<int64_t> host(num_tokens);
    if (hipStreamSynchronize(stream) != hipSuccess ||
        hipMemcpy(host.data(), slot_mapping, sizeof(int64_t) * num_tokens,
                  hipMemcpyDeviceToHost) != hipSuccess)
      return PKV_ERR_HIP;
    std::vector<char> seen(num_slots, 0);
    for (int64_t s : host) {
      if (s < 0) continue;
      if (s >= num_slots || seen[s]) return PKV_ERR_INVALID;
      seen[s] = 1;
    }
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

pkv_status paged_kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs,
                                int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                                int32_t num_blocks, pkv_dtype dtype, hipStream_t stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0)
    return PKV_ERR_INVALID;
  if (head_dim % 32 != 0 || elem_size(dtype) == 0) return PKV_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !pairs) return PKV_ERR_INVALID;
  const int64_t run_bytes = int64_t(num_kv_heads) * kBlock * head_dim * elem_size(dtype);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, 2), dim3(256), 0, stream,
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), pairs,
                     run_bytes / 16, num_blocks);
  return launch_status();
}

size_t paged_attention_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                      int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || partition_size < 0) return 0;
  const int part = resolve_partition(partition_size);
  const int64_t mp = max_parts_for(max_context_len, part);
  if (mp <= 1) return 0;
  return size_t(num_seqs) * num_q_heads * mp * (head_dim + 2) * sizeof(float);
}

pkv_status paged_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t num_blocks,
                                  int32_t max_blocks_per_seq, int32_t max_context_len,
                                  float scale, int32_t partition_size, void* workspace,
                                  size_t workspace_bytes, pkv_dtype kv_dtype, float* out,
                                  hipStream_t stream) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_blocks <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0 || partition_size < 0)
    return PKV_ERR_INVALID;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_INVALID;
  if (partition_size % 32 != 0) return PKV_ERR_INVALID;
  if (num_seqs > 65535 || num_kv_heads > 65535 || num_q_heads > 65535) return PKV_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (elem_size(kv_dtype) == 0) return PKV_ERR_UNSUPPORTED;
  const int group = num_q_heads / num_kv_heads;
  if (kv_dtype == PKV_BF16 && group > 16) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return PKV_ERR_INVALID;
  const int part = resolve_partition(partition_size);
  const int64_t max_parts = max_parts_for(max_context_len, part);
  if (max_parts > 65535) return PKV_ERR_UNSUPPORTED;
  const size_t need = paged_attention_workspace_size(num_seqs, num_q_heads, head_dim,
                                                     max_context_len, partition_size);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_ERR_INVALID;

  DecodeArgs a;
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.out = out;
  const int64_t heads = int64_t(num_seqs) * num_q_heads;
  float* ws = static_cast<float*>(workspace);
  a.ws_o = ws;
  a.ws_m = ws ? ws + heads * max_parts * head_dim : nullptr;
  a.ws_l = ws ? a.ws_m + heads * max_parts : nullptr;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.max_ctx = max_context_len;
  a.part_tokens = part;
  a.max_parts = static_cast<int>(max_parts);
  a.scale_log2e = scale * 1.4426950408889634f;

  const bool prof = g_prof.on && g_prof.used + 2 <= g_prof.pool.size();
  if (prof) (void)hipEventRecord(g_prof.pool[g_prof.used], stream);
  if (kv_dtype == PKV_BF16) {
    dim3 grid(static_cast<unsigned>(max_parts), num_kv_heads, num_seqs);
    if (head_dim == 128)
      hipLaunchKernelGGL(decode_bf16_kernel<128>, grid, dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL(decode_bf16_kernel<64>, grid, dim3(64), 0, stream, a);
  } else {
    dim3 grid(static_cast<unsigned>(max_parts), num_q_heads, num_seqs);
    if (head_dim == 128)
      hipLaunchKernelGGL(decode_f32_kernel<128>, grid, dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL(decode_f32_kernel<64>, grid, dim3(64), 0, stream, a);
  }
  if (prof) {
    (void)hipEventRecord(g_prof.pool[g_prof.used + 1], stream);
    g_prof.used += 2;
  }
  pkv_status st = launch_status();
  if (st != PKV_OK || max_parts <= 1) return st;
  const unsigned rgrid = static_cast<unsigned>(heads);
  if (head_dim == 128)
    hipLaunchKernelGGL(lse_reduce_kernel<128>, dim3(rgrid), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL(lse_reduce_kernel<64>, dim3(rgrid), dim3(64), 0, stream, a);
  return launch_status();
}

pkv_status pkv_profile_begin(void) {
  if (g_prof.pool.empty()) {
    g_prof.pool.resize(2 * kMaxProfiled);
    for (auto& e : g_prof.pool)
      if (hipEventCreate(&e) != hipSuccess) {
        g_prof.pool.clear();
        return PKV_ERR_HIP;
      }
  }
  g_prof.used = 0;
  g_prof.on = true;
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
