// Selective attention of the recomputed rows (pic_selective_attn).
//
// EPIC walkthrough, link_legolink Step 3: the recomputed rows' Q, rotated at their
// global positions, attend over the spliced K/V with a causal mask.  For a row at
// position p the visible keys are j <= p, which is the offset mask of "KV cache 从零
// 实现" (allowed[i, j] = [j <= P + i] for a run of rows starting at P).  GQA maps
// query head h to KV head h / G.
//
// Work decomposition (the host planner builds it): an attention tile is
// PIC_ATTN_TILE_M = 128 query vectors -- 128/G consecutive recomputed rows of one
// request times the G query heads that share one KV head -- so every K/V element
// staged in LDS feeds 128 query vectors.  An item is (tile, kv head, key range); long
// tiles are split along keys and a merge kernel combines the partial results with
// their log-sum-exp weights.
//
// The math is the flash-attention recurrence in transposed form: S^T = K Q^T puts one
// query per MFMA output column, so a lane holds many keys of one query and the softmax
// statistics need one (32x32 tiles) or two (16x16 tiles) cross-lane exchanges; then
// O^T += V^T P^T consumes the probabilities straight from the S^T registers.  Rows of
// the K operand are permuted so that each lane's probabilities are exactly the
// consecutive keys its PV operand slots need.  The running max is kept in the exp2
// domain (scores scaled by scale * log2 e).
//
// bf16 kernel (the hot one): 4 waves x 32 queries, v_mfma_f32_32x32x16_bf16 for both
// products, K/V blocks of 64 keys double-buffered in LDS and staged by direct
// buffer->LDS loads (the buffer range clamps rows past the item's keys to zero), K
// one block ahead of V so that S^T of block i+1 is computed while block i's softmax
// runs (software pipelining inside each wave), V read transposed for
// the PV operand with ds_read_b64_tr_b16, row sums taken from the bf16 probabilities
// with v_dot2_f32_bf16.
// fp32 kernel: 8 waves x 16 queries, v_mfma_f32_16x16x4_f32 (fp32 operands, so fp32
// I/O keeps fp32 accuracy), V staged transposed.
#include <algorithm>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "pic_device.h"
#include "pic_internal.h"

namespace pic {
namespace {

constexpr int kM = PIC_ATTN_TILE_M;  // query vectors per tile
constexpr int kKB = 64;              // keys per staged block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bool wave_any(bool p) { return __any((int)p); }

// max / sum of a value over the lane pair (l, l ^ 32), in the VALU (v_permlane32_swap)
__device__ __forceinline__ float pair_max(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// The lane id, produced afresh at each call (an opaque instruction pair the compiler
// cannot merge with another), so values derived from it on a rarely taken path are
// recomputed there instead of being held across the main loop: in a kernel at the
// register limit such values get spilled, and reloading a spill is a vector memory load
// whose wait also waits for every direct load issued before it.
__device__ __forceinline__ int fresh_lane() {
  int v;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
  return v;
}

// ================================ bf16 kernel ==================================

constexpr int kBfWaves = 4;
constexpr int kBfThreads = 64 * kBfWaves;
static_assert(kM == 32 * kBfWaves, "one 32-query MFMA column block per wave");

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

// Key (0..31 within a 32-key S^T tile t of the 64-key block) at C row r: rows held by
// lane group g in accumulator slots 8h..8h+7 become keys 16(2t+h) + 8g + 0..7.
__device__ __forceinline__ int perm_key(int t, int r) {
  const int a = r >> 3, g = (r >> 2) & 1, b = r & 3;
  return 16 * (2 * t + (a >> 1)) + 8 * g + 4 * (a & 1) + b;
}

// LDS layouts: a staged block is 64 key rows of D bf16, rows unpadded, 16-byte chunks
// XOR-swizzled per row so that the reads of one LDS cycle hit distinct banks.
// K rows are read 16 at a time (rows {0..3, 8..11, 16..19, 24..27} + const, one chunk
// each): the swizzle takes 16 distinct values over such a set.  V rows are read by the
// transposing loads 4 consecutive rows at a time, two lane groups on adjacent chunk
// pairs: XOR of chunk bits 2-3 by (row & 3) puts the four rows on four distinct
// 64-byte bank groups.
template <int kCPR>
__device__ __forceinline__ int swz_k(int r) {
  return ((r & 3) | (((r >> 3) & 3) << 2)) & (kCPR - 1);
}
template <int kCPR>
__device__ __forceinline__ int swz_v(int r) {
  return (4 * (r & 3)) & (kCPR - 1);
}

template <int D>
__device__ __forceinline__ void attn_bf16_body(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ kbuf,
    const __bf16 *__restrict__ vbuf, __bf16 *__restrict__ out, const int32_t *__restrict__ rows,
    const AttnTile *__restrict__ tiles, const AttnItem *__restrict__ items,
    float *__restrict__ ws_o, float *__restrict__ ws_ml, int h_q, int h_kv, int tile_rows,
    float scale_log2) {
  constexpr int kRowB = D * 2;                 // bytes per staged key row
  constexpr int kCPR = D / 8;                  // 16-byte chunks per row
  constexpr int kTileB = kKB * kRowB;          // bytes of one staged K or V block
  constexpr int kRPI = 1024 / kRowB;           // rows one wave fills per direct load
  constexpr int kRounds = kKB / (kRPI * kBfWaves);  // direct loads per wave per tensor
  constexpr int kKS = D / 16;                  // S^T contraction steps
  constexpr int kDB = D / 32;                  // 32-wide d blocks of O^T
  static_assert(kRounds * kRPI * kBfWaves == kKB, "direct loads must tile the block");
  static_assert(2 * kKS <= 16, "S^T MFMAs of a block must fit the 16 exponential pairs");
  // [buffer 0: K, V][buffer 1: K, V]
  __shared__ __attribute__((aligned(1024))) char lds[4 * kTileB];

  const AttnItem it = items[blockIdx.x];
  const AttnTile tile = tiles[it.tile];
  const int g = it.kv_head;
  const int group = h_q / h_kv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31;     // query column of this lane
  const int grp = lane >> 5;   // lane group (0, 1)
  const int q16 = lane >> 4;   // 16-lane group of the transposing read
  const int i16 = lane & 15;

  const int m = 32 * wave + n;
  const int row_local = m % tile_rows;
  const int head = g * group + m / tile_rows;
  const bool valid = row_local < tile.n_rows;
  const int row = tile.row_begin + (valid ? row_local : 0);
  const int pos = valid ? rows[row] : -1;

  bf16x8 qop[kKS];
  {
    const __bf16 *qp = q + ((int64_t)row * h_q + head) * D + 8 * grp;
#pragma unroll
    for (int s = 0; s < kKS; ++s)
      qop[s] = valid ? *reinterpret_cast<const bf16x8 *>(qp + 16 * s) : bf16x8{};
  }
  int pos_min = valid ? pos : 0x7fffffff;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) pos_min = min(pos_min, __shfl_xor(pos_min, o));

  f32x16 acc[kDB];
#pragma unroll
  for (int d = 0; d < kDB; ++d)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[d][j] = 0.f;
  float m_run = kNegInf;
  float l_lane = 0.f;

  const int key_begin = it.key_begin;
  const int key_end = it.key_end;
  const int key_last = key_end - 1;
  const int tok_bytes = h_kv * D * 2;

  // ---- direct global->LDS staging: buffer resources clamp rows >= key_end to zero ----
  // (the resources are rebuilt where used: a lambda may not capture the resource type;
  // the block's row offset rides in the per-lane offset, which the range check sees)
  const int64_t head_off = ((int64_t)tile.tok_base * h_kv + g) * D;
  const __bf16 *kh = kbuf + head_off;
  const __bf16 *vh = vbuf + head_off;
  const int n_records = key_end * tok_bytes;
  int voff_k[kRounds], voff_v[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int R = kRPI * (kBfWaves * r + wave) + lane / kCPR;  // block row this lane fills
    const int p = lane % kCPR;                                 // its physical chunk
    voff_k[r] = R * tok_bytes + 16 * (p ^ swz_k<kCPR>(R));
    voff_v[r] = R * tok_bytes + 16 * (p ^ swz_v<kCPR>(R));
  }
  // LDS: K blocks in buffers 0/1, V blocks in buffers 2/3.  K is staged one block
  // ahead of V so that S^T of block i+1 can be computed while block i's softmax runs.
  auto issue = [&](const __bf16 *base, const int (&voffs)[kRounds], int kb0, int buf) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, n_records, 0x00020000);
    // unsigned: rows past the request's end may lie past 2^31 bytes (read as zeros)
    const unsigned first = (unsigned)kb0 * (unsigned)tok_bytes;
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int dst = buf * kTileB + (kBfWaves * r + wave) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(lds + dst), 16,
                                               (int)((unsigned)voffs[r] + first), 0, 0, 0);
    }
  };

  // ---- loop-invariant LDS read offsets (bytes within a K or V block) ----
  int koff[kKS];
  {
    const int r0 = perm_key(0, n);  // tile 1 is rows + 32, same swizzle
    const int f = swz_k<kCPR>(r0);
#pragma unroll
    for (int s = 0; s < kKS; ++s) koff[s] = r0 * kRowB + 16 * ((2 * s + grp) ^ f);
  }
  int voff[kDB];
  {
    const int rr = 8 * (q16 >> 1) + (i16 >> 2);  // + 16c + 4h, which keeps rr & 3
    const int f = swz_v<kCPR>(rr) >> 2;
#pragma unroll
    for (int d = 0; d < kDB; ++d)
      voff[d] = rr * kRowB + 16 * (4 * (d ^ f) + 2 * (q16 & 1) + ((i16 & 3) >> 1)) +
                8 * (i16 & 1);
  }

  // S^T = K Q^T for the two 32-key tiles of the block in K buffer kb.
  auto qk = [&](const char *Kb, f32x16 (&sc)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int j = 0; j < 16; ++j) sc[t][j] = 0.f;
#pragma unroll
      for (int s = 0; s < kKS; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(Kb + koff[s] + t * 32 * kRowB);
        sc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[s], sc[t], 0, 0, 0);
      }
    }
  };

  // Mask, online softmax and O^T += V^T P^T for the block starting at key kb0; S^T of
  // the next block (K buffer Knext) is computed into s_nxt meanwhile, its 16 MFMAs
  // interleaved with the 32 exponentials and each K operand read eight MFMAs ahead
  // (after the last block the result is unused); the PV MFMAs read their transposed V
  // operands two ahead as well.  The running max m_run is only moved when a
  // column's block max exceeds it by more than kLazy (log2 units), so rescaling the
  // accumulators is rare; probabilities then stay below 2^kLazy, far inside fp32/bf16
  // range, and the final normalisation is unchanged (acc and l share the reference).
  auto softmax_pv = [&](f32x16 (&sc)[2], int kb0, const char *Vb, const char *Knext,
                        f32x16 (&s_nxt)[2]) {
    constexpr float kLazy = 8.f;
    if (kb0 + kKB - 1 > min(pos_min, key_last)) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = kb0 + perm_key(t, 8 * (j >> 2) + 4 * grp + (j & 3));
          if (key > pos || key > key_last) sc[t][j] = kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sc[t][j]);
    mx = pair_max(mx) * scale_log2;
    const bool upd = mx > m_run + kLazy;  // false while everything seen is masked
    if (wave_any(upd)) {
      const float alpha = upd ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
      m_run = upd ? mx : m_run;
      l_lane *= alpha;
#pragma unroll
      for (int d = 0; d < kDB; ++d) acc[d] *= alpha;
    }
    const float base = m_run == kNegInf ? 0.f : m_run;

    bf16x8 pb[4];
    const bf16x2v ones = {(__bf16)1.f, (__bf16)1.f};
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) s_nxt[t][j] = 0.f;
    constexpr int kPre = 8;  // K operand reads in flight ahead of their MFMA
    bf16x8 kop[2 * kKS];
    auto kload = [&](int q) {
      kop[q] = *reinterpret_cast<const bf16x8 *>(Knext + koff[q >> 1] + (q & 1) * 32 * kRowB);
    };
#pragma unroll
    for (int q = 0; q < kPre; ++q) kload(q);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (q < 2 * kKS) {  // S^T MFMAs of the next block, one per pair; tiles alternate
        if (q + kPre < 2 * kKS) kload(q + kPre);
        const int t = q & 1, s = q >> 1;
        s_nxt[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[q], qop[s], s_nxt[t], 0, 0, 0);
      }
      const int t = q >> 3, j = 2 * (q & 7);
      bf16x2v pr;
      pr[0] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[t][j], scale_log2, -base));
      pr[1] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[t][j + 1], scale_log2, -base));
      pb[2 * t + (j >> 3)][j & 7] = pr[0];
      pb[2 * t + (j >> 3)][(j & 7) + 1] = pr[1];
      if (j & 2) ps1 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ps1, false);
      else ps0 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ps0, false);
    }
    // keep the schedule interleaved: per pair, its K read, one MFMA, the VALU work
#pragma unroll
    for (int q = 0; q < kPre; ++q) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int q = 0; q < 2 * kKS; ++q) {
      if (q + kPre < 2 * kKS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
    }
    l_lane += ps0 + ps1;
    __builtin_amdgcn_s_setprio(1);
    constexpr int kPreV = 2;  // V operands in flight ahead of their MFMA
    bf16x8 vop[4 * kDB];
    auto vload = [&](int o) {
      const char *vr = Vb + voff[o % kDB] + (o / kDB) * 16 * kRowB;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)vr);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vr + 4 * kRowB));
      __builtin_memcpy(&vop[o], &lo, 8);
      __builtin_memcpy(reinterpret_cast<char *>(&vop[o]) + 8, &hi, 8);
    };
#pragma unroll
    for (int o = 0; o < kPreV; ++o) vload(o);
#pragma unroll
    for (int o = 0; o < 4 * kDB; ++o) {
      if (o + kPreV < 4 * kDB) vload(o + kPreV);
      acc[o % kDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[o], pb[o / kDB], acc[o % kDB], 0, 0, 0);
    }
#pragma unroll
    for (int o = 0; o < kPreV; ++o) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int o = 0; o < 4 * kDB; ++o) {
      if (o + kPreV < 4 * kDB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  const int n_blocks = (key_end - key_begin + kKB - 1) / kKB;
  issue(kh, voff_k, key_begin, 0);
  issue(vh, voff_v, key_begin, 2);
  if (n_blocks > 1) issue(kh, voff_k, key_begin + kKB, 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  f32x16 sa[2], sb[2];
  qk(lds, sa);
  __syncthreads();  // K buffer 0 is refilled next

  // Block ib: S^T(ib) is in registers; stage K(ib+2) and V(ib+1), compute S^T(ib+1),
  // then the softmax and PV of block ib.  kB = ib & 1 selects the buffers.
  auto step = [&](int ib, auto bufc, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2]) {
    constexpr int kB = decltype(bufc)::value;
    const int kb0 = key_begin + ib * kKB;
    if (ib + 2 < n_blocks) issue(kh, voff_k, kb0 + 2 * kKB, kB);
    if (ib + 1 < n_blocks) issue(vh, voff_v, kb0 + kKB, 2 + (kB ^ 1));
    softmax_pv(s_cur, kb0, lds + (2 + kB) * kTileB, lds + (kB ^ 1) * kTileB, s_nxt);
    if (ib + 1 < n_blocks) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
  };

  for (int ib = 0; ib < n_blocks; ib += 2) {
    step(ib, std::integral_constant<int, 0>{}, sa, sb);
    if (ib + 1 < n_blocks) step(ib + 1, std::integral_constant<int, 1>{}, sb, sa);
  }

  // ---- epilogue ----
  const float l_row = pair_sum(l_lane);
  if (!valid) return;
  if (it.slot < 0) {
    const float inv = 1.f / l_row;
    __bf16 *op = out + ((int64_t)row * h_q + head) * D + 4 * grp;
#pragma unroll
    for (int d = 0; d < kDB; ++d)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 o;
#pragma unroll
        for (int b = 0; b < 4; ++b) o[b] = (__bf16)(acc[d][4 * a + b] * inv);
        *reinterpret_cast<bf16x4 *>(op + 32 * d + 8 * a) = o;
      }
  } else {
    __bf16 *wo = reinterpret_cast<__bf16 *>(ws_o) + ((int64_t)it.slot * kM + m) * D + 4 * grp;
#pragma unroll
    for (int d = 0; d < kDB; ++d)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 o;
#pragma unroll
        for (int b = 0; b < 4; ++b) o[b] = (__bf16)acc[d][4 * a + b];
        *reinterpret_cast<bf16x4 *>(wo + 32 * d + 8 * a) = o;
      }
    if (grp == 0) {
      ws_ml[((int64_t)it.slot * kM + m) * 2 + 0] = m_run;
      ws_ml[((int64_t)it.slot * kM + m) * 2 + 1] = l_row;
    }
  }
}

template <int D>
__global__ __launch_bounds__(kBfThreads, 2) void attn_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ kbuf,
    const __bf16 *__restrict__ vbuf, __bf16 *__restrict__ out, const int32_t *__restrict__ rows,
    const AttnTile *__restrict__ tiles, const AttnItem *__restrict__ items,
    float *__restrict__ ws_o, float *__restrict__ ws_ml, int h_q, int h_kv, int tile_rows,
    float scale_log2) {
  attn_bf16_body<D>(q, kbuf, vbuf, out, rows, tiles, items, ws_o, ws_ml, h_q, h_kv, tile_rows,
                    scale_log2);
}

// ============================ bf16 kernel, paged pool ===========================
//
// Chunks are stored once in a shared pool of 16-row blocks, so cached K cannot be
// rotated in place.  Instead each chunk's keys are scored in their local RoPE frame
// against the query rotated the other way: <q, R(delta_c) k> = <R(-delta_c) q, k>
// (rotations are orthogonal), once per chunk per wave.  The recomputed rows (seams and
// queries) are read straight from the fresh buffers in the global frame, as their own
// key blocks; the online softmax does not depend on key order.  Every staged block
// therefore comes from one buffer, so direct buffer->LDS loads still apply: a 64-key
// block's four 16-row pool blocks come from a per-block record that a small kernel
// resolves from the block table before the attention kernel runs, rows past a chunk's
// last block read as zero, and V rows past a chunk's end are zeroed in LDS so that
// masked keys contribute exactly nothing.

constexpr int kPoolBlockRows = 16;

// cos/sin(delta_c * theta_i) for every chunk c and pair i of the plan.
__global__ __launch_bounds__(256) void paged_angles_kernel(float2 *__restrict__ angles,
                                                           const int32_t *__restrict__ segs,
                                                           int n_chunks, int n_pairs,
                                                           ThetaTable theta) {
  const int64_t total = (int64_t)n_chunks * n_pairs;
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * 256) {
    const int c = (int)(u / n_pairs), i = (int)(u - (int64_t)c * n_pairs);
    angles[u] = delta_cos_sin(segs[8 * c + 4], theta.hi[i], theta.lo[i]);
  }
}

// Everything the attention kernel needs to stage and mask one 64-key block, resolved
// once per launch so that the kernel reads a single 32-byte record per block (one
// scalar load) instead of walking segment -> chunk -> block table with dependent loads.
struct KeyBlockRec {
  int32_t frame;     // global chunk index c (its angle row), or -1: the request's fresh rows
  int32_t row;       // fresh: first fresh row of the block; pool: first local key t0
  int32_t base_pos;  // pool: global position of local key t0
  int32_t vis;       // pool: visible local keys [s0, nv) of the block as s0 | nv << 8
  int32_t off[4];    // pool: byte offset of each 16-row pool block, -1: reads zeros
};
static_assert(sizeof(KeyBlockRec) == 32, "one s_load_dwordx8 per record");
static_assert(kKB == 4 * kPoolBlockRows, "a key block spans four pool blocks");

__global__ __launch_bounds__(256) void paged_blocks_kernel(
    KeyBlockRec *__restrict__ recs, const int4 *__restrict__ kblocks,
    const int32_t *__restrict__ segs, const int32_t *__restrict__ chunk_block_ptr,
    const int32_t *__restrict__ block_ids, int n_kblocks, int pool_blocks, int blk_bytes) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n_kblocks) return;
  const int4 d = kblocks[i];
  KeyBlockRec r;
  r.frame = d.x;
  r.row = d.y;
  if (d.x < 0) {
    r.base_pos = 0;
    r.vis = kKB << 8;
#pragma unroll
    for (int b = 0; b < 4; ++b) r.off[b] = -1;
  } else {
    const int32_t *sg = segs + 8 * d.x;
    const int off = sg[0], len = sg[1], seam = sg[2], cid = sg[3];
    // blocks the chunk needs, bounded by the blocks its table row lists: an undersized
    // row reads zeros past its end instead of the next chunk's ids (or past the table)
    const int tab0 = chunk_block_ptr[cid];
    const int nb = min((len + kPoolBlockRows - 1) / kPoolBlockRows,
                       max(0, chunk_block_ptr[cid + 1] - tab0));
    const int32_t *bl = block_ids + tab0;
    r.base_pos = off + d.y;
    r.vis = max(0, min(kKB, seam - d.y)) | (min(kKB, len - d.y) << 8);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int pb = d.y / kPoolBlockRows + b;
      const int bid = pb < nb ? bl[pb] : -1;
      r.off[b] = (unsigned)bid < (unsigned)pool_blocks ? bid * blk_bytes : -1;
    }
  }
  recs[i] = r;
}

template <int D, bool kHalf>
__device__ __forceinline__ void attn_bf16_paged_body(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ pool_k,
    const __bf16 *__restrict__ pool_v, const __bf16 *__restrict__ k_fresh,
    const __bf16 *__restrict__ v_fresh, __bf16 *__restrict__ out,
    const int32_t *__restrict__ rows, const AttnTile *__restrict__ tiles,
    const AttnItem *__restrict__ items, const KeyBlockRec *__restrict__ recs,
    const float2 *__restrict__ angles, float *__restrict__ ws_o, float *__restrict__ ws_ml,
    int h_q, int h_kv, int tile_rows, float scale_log2, int pool_bytes) {
  constexpr int kRowB = D * 2;
  constexpr int kCPR = D / 8;
  constexpr int kTileB = kKB * kRowB;
  constexpr int kRPI = 1024 / kRowB;
  constexpr int kRounds = kKB / (kRPI * kBfWaves);
  constexpr int kKS = D / 16;
  constexpr int kDB = D / 32;
  constexpr int kPairs = D / 2;
  static_assert(kRounds * kRPI * kBfWaves == kKB, "direct loads must tile the block");
  static_assert(2 * kKS <= 16, "S^T MFMAs of a block must fit the 16 exponential pairs");
  static_assert(kRPI <= kPoolBlockRows, "one direct load must stay inside a pool block");
  __shared__ __attribute__((aligned(1024))) char lds[4 * kTileB];
  __shared__ int kpos[2][kKB];  // key positions of fresh blocks (INT_MAX: no key)

  const AttnItem it = items[blockIdx.x];
  const AttnTile tile = tiles[it.tile];
  const int g = it.kv_head;
  const int group = h_q / h_kv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31;
  const int grp = lane >> 5;
  const int q16 = lane >> 4;
  const int i16 = lane & 15;

  const int m = 32 * wave + n;
  const int row_local = m % tile_rows;
  const int head = g * group + m / tile_rows;
  const bool valid = row_local < tile.n_rows;
  const int row = tile.row_begin + (valid ? row_local : 0);
  const int pos = valid ? rows[row] : -1;
  const int fresh_base = tile.pad0, n_fresh = tile.pad1;

  int pos_min = valid ? pos : 0x7fffffff;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) pos_min = min(pos_min, __shfl_xor(pos_min, o));

  // ---- query operand in the frame of the block being scored ----
  bf16x8 qop[kKS];
  int frame = -2;  // -1: global frame (fresh keys); c >= 0: local frame of chunk c
  const __bf16 *qp = q + ((int64_t)row * h_q + head) * D + 8 * grp;
  auto set_frame = [&](int f) {
    if (f == frame) return;
    frame = f;
    bf16x8 qo[kKS];
#pragma unroll
    for (int s = 0; s < kKS; ++s)
      qo[s] = valid ? *reinterpret_cast<const bf16x8 *>(qp + 16 * s) : bf16x8{};
    if (f < 0) {
#pragma unroll
      for (int s = 0; s < kKS; ++s) qop[s] = qo[s];
      return;
    }
    const float2 *cs = angles + (int64_t)f * kPairs;  // rotate by -delta_c
    if constexpr (!kHalf) {
#pragma unroll
      for (int s = 0; s < kKS; ++s)
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const float2 c = cs[8 * s + 4 * grp + j / 2];
          const float a = (float)qo[s][j], b = (float)qo[s][j + 1];
          qop[s][j] = (__bf16)(a * c.x + b * c.y);
          qop[s][j + 1] = (__bf16)(b * c.x - a * c.y);
        }
    } else {
#pragma unroll
      for (int s = 0; s < kKS / 2; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float2 c = cs[16 * s + 8 * grp + j];
          const float a = (float)qo[s][j], b = (float)qo[s + kKS / 2][j];
          qop[s][j] = (__bf16)(a * c.x + b * c.y);
          qop[s + kKS / 2][j] = (__bf16)(b * c.x - a * c.y);
        }
    }
  };

  f32x16 acc[kDB];
#pragma unroll
  for (int d = 0; d < kDB; ++d)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[d][j] = 0.f;
  float m_run = kNegInf;
  float l_lane = 0.f;

  // ---- key blocks: item ranges [key_begin, key_end) then [pad0, pad1) ----
  const int n1 = it.key_end - it.key_begin;
  const int n_blocks = n1 + (it.pad1 - it.pad0);
  auto desc = [&](int ib) { return recs[ib < n1 ? it.key_begin + ib : it.pad0 + ib - n1]; };

  const int tok_bytes = h_kv * D * 2;
  const __bf16 *kfh = k_fresh + ((int64_t)fresh_base * h_kv + g) * D;
  const __bf16 *vfh = v_fresh + ((int64_t)fresh_base * h_kv + g) * D;
  // per-lane byte offsets of the row and chunk each lane stages, relative to the block's
  // first row (K and V swizzles); everything uniform goes into the resource's base
  int voff_k[kRounds], voff_v[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int R = kRPI * (kBfWaves * r + wave) + lane / kCPR;
    const int pch = lane % kCPR;
    voff_k[r] = R * tok_bytes + 16 * (pch ^ swz_k<kCPR>(R));
    voff_v[r] = R * tok_bytes + 16 * (pch ^ swz_v<kCPR>(R));
  }

  // Stage one K (is_v = false) or V block into LDS buffer `buf` (direct loads).  The
  // resource's base is the block's first row, so the per-lane offsets are the same for
  // every block.  Fresh rows: the range (rows left in the fresh buffer) clamps rows past
  // them to zero.  Pool rows: the load of rows r0 .. r0 + kRPI - 1 (one 16-row pool block)
  // gets that pool block's row 0 minus r0 rows as its base, so the same per-lane offsets
  // land in it; a pool block past the chunk's end or outside the pool (offset -1) gets a
  // resource of zero records (zeros), any other lies wholly inside the pool.
  auto issue = [&](const KeyBlockRec &dsc, bool is_v, int buf) {
    const int *vo = is_v ? voff_v : voff_k;
    if (dsc.frame < 0) {
      const char *base =
          reinterpret_cast<const char *>(is_v ? vfh : kfh) + (int64_t)dsc.row * tok_bytes;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void *)base, 0, (n_fresh - dsc.row) * tok_bytes, 0x00020000);
#pragma unroll
      for (int r = 0; r < kRounds; ++r) {
        const int dst = buf * kTileB + (kBfWaves * r + wave) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(lds + dst), 16, vo[r], 0, 0, 0);
      }
    } else {
      const char *pool = reinterpret_cast<const char *>(is_v ? pool_v : pool_k) + g * kRowB;
#pragma unroll
      for (int r = 0; r < kRounds; ++r) {
        const int r0 = kRPI * (kBfWaves * r + wave) / kPoolBlockRows * kPoolBlockRows;
        const int pl = r0 / kPoolBlockRows;  // uniform, 0..3
        const int o = pl == 0 ? dsc.off[0] : pl == 1 ? dsc.off[1] : pl == 2 ? dsc.off[2] : dsc.off[3];
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(pool + (int64_t)o - (int64_t)r0 * tok_bytes), 0, o >= 0 ? 0x7fffffff : 0,
            0x00020000);
        const int dst = buf * kTileB + (kBfWaves * r + wave) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(lds + dst), 16, vo[r], 0, 0, 0);
      }
    }
  };
  // After a V block landed: zero V rows past the chunk's end (pool blocks) and record
  // key positions (fresh blocks).  Both are rare (a chunk's last block, the fresh
  // blocks): the lane-derived values and the zero are made here (fresh_lane).
  auto finish_v = [&](const KeyBlockRec &dsc, int buf) {
    if (dsc.frame < 0) {
      if (wave == 0) {
        const int ln = fresh_lane();
        const int r = dsc.row + ln;
        kpos[buf & 1][ln] = r < n_fresh ? rows[fresh_base + r] : 0x7fffffff;
      }
      return;
    }
    const int nv = dsc.vis >> 8;
    if (nv >= kKB) return;
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int ln = fresh_lane();
      const int R = kRPI * (kBfWaves * r + wave) + ln / kCPR;
      if (R >= nv) {
        const int dst = (2 + buf) * kTileB + (kBfWaves * r + wave) * 1024 + 16 * ln;
        unsigned z;
        asm volatile("v_mov_b32 %0, 0" : "=v"(z));
        *reinterpret_cast<u32x4 *>(lds + dst) = u32x4{z, z, z, z};
      }
    }
  };

  int koff[kKS];
  {
    const int r0 = perm_key(0, n);
    const int f = swz_k<kCPR>(r0);
#pragma unroll
    for (int s = 0; s < kKS; ++s) koff[s] = r0 * kRowB + 16 * ((2 * s + grp) ^ f);
  }
  int voff[kDB];
  {
    const int rr = 8 * (q16 >> 1) + (i16 >> 2);
    const int f = swz_v<kCPR>(rr) >> 2;
#pragma unroll
    for (int d = 0; d < kDB; ++d)
      voff[d] = rr * kRowB + 16 * (4 * (d ^ f) + 2 * (q16 & 1) + ((i16 & 3) >> 1)) +
                8 * (i16 & 1);
  }

  auto qk = [&](const char *Kb, f32x16 (&sc)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int j = 0; j < 16; ++j) sc[t][j] = 0.f;
#pragma unroll
      for (int s = 0; s < kKS; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(Kb + koff[s] + t * 32 * kRowB);
        sc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[s], sc[t], 0, 0, 0);
      }
    }
  };

  auto softmax_pv = [&](f32x16 (&sc)[2], const KeyBlockRec &dsc, int buf, const char *Knext,
                        f32x16 (&s_nxt)[2]) {
    constexpr float kLazy = 8.f;
    const char *Vb = lds + (2 + buf) * kTileB;
    if (dsc.frame < 0) {  // fresh keys: positions from LDS
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int kp = kpos[buf][perm_key(t, 8 * (j >> 2) + 4 * grp + (j & 3))];
          if (kp > pos) sc[t][j] = kNegInf;
        }
    } else {
      const int s0 = dsc.vis & 255, nv = dsc.vis >> 8;
      if (s0 > 0 || nv < kKB || dsc.base_pos + kKB - 1 > pos_min) {
        const int lim = min(nv, pos - dsc.base_pos + 1);  // block keys [s0, lim) are visible
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int tk = perm_key(t, 8 * (j >> 2) + 4 * grp + (j & 3));
            if (tk < s0 || tk >= lim) sc[t][j] = kNegInf;
          }
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sc[t][j]);
    mx = pair_max(mx) * scale_log2;
    const bool upd = mx > m_run + kLazy;
    if (wave_any(upd)) {
      const float alpha = upd ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
      m_run = upd ? mx : m_run;
      l_lane *= alpha;
#pragma unroll
      for (int d = 0; d < kDB; ++d) acc[d] *= alpha;
    }
    const float base = m_run == kNegInf ? 0.f : m_run;
    bf16x8 pb[4];
    const bf16x2v ones = {(__bf16)1.f, (__bf16)1.f};
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) s_nxt[t][j] = 0.f;
    constexpr int kPre = 2;  // K operand reads in flight ahead of their MFMA
    bf16x8 kop[2 * kKS];
    auto kload = [&](int q) {
      kop[q] = *reinterpret_cast<const bf16x8 *>(Knext + koff[q >> 1] + (q & 1) * 32 * kRowB);
    };
#pragma unroll
    for (int q = 0; q < kPre; ++q) kload(q);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (q < 2 * kKS) {
        if (q + kPre < 2 * kKS) kload(q + kPre);
        const int t = q & 1, s = q >> 1;
        s_nxt[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[q], qop[s], s_nxt[t], 0, 0, 0);
      }
      const int t = q >> 3, j = 2 * (q & 7);
      bf16x2v pr;
      pr[0] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[t][j], scale_log2, -base));
      pr[1] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[t][j + 1], scale_log2, -base));
      pb[2 * t + (j >> 3)][j & 7] = pr[0];
      pb[2 * t + (j >> 3)][(j & 7) + 1] = pr[1];
      if (j & 2) ps1 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ps1, false);
      else ps0 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ps0, false);
    }
#pragma unroll
    for (int q = 0; q < kPre; ++q) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int q = 0; q < 2 * kKS; ++q) {
      if (q + kPre < 2 * kKS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    }
    l_lane += ps0 + ps1;
    __builtin_amdgcn_s_setprio(1);
    constexpr int kPreV = 2;  // V operands in flight ahead of their MFMA
    bf16x8 vop[4 * kDB];
    auto vload = [&](int o) {
      const char *vr = Vb + voff[o % kDB] + (o / kDB) * 16 * kRowB;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)vr);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vr + 4 * kRowB));
      __builtin_memcpy(&vop[o], &lo, 8);
      __builtin_memcpy(reinterpret_cast<char *>(&vop[o]) + 8, &hi, 8);
    };
#pragma unroll
    for (int o = 0; o < kPreV; ++o) vload(o);
#pragma unroll
    for (int o = 0; o < 4 * kDB; ++o) {
      if (o + kPreV < 4 * kDB) vload(o + kPreV);
      acc[o % kDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[o], pb[o / kDB], acc[o % kDB], 0, 0, 0);
    }
#pragma unroll
    for (int o = 0; o < kPreV; ++o) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int o = 0; o < 4 * kDB; ++o) {
      if (o + kPreV < 4 * kDB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- prologue: K(0), V(0), K(1) ----
  KeyBlockRec d0 = desc(0);
  issue(d0, false, 0);
  issue(d0, true, 2);
  KeyBlockRec d1 = n_blocks > 1 ? desc(1) : d0;
  if (n_blocks > 1) issue(d1, false, 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  finish_v(d0, 0);
  __syncthreads();
  f32x16 sa[2], sb[2];
  set_frame(d0.frame);
  qk(lds, sa);
  __syncthreads();

  // Block ib: S^T(ib) is in registers; stage K(ib+2) and V(ib+1), compute S^T(ib+1) in
  // block ib+1's frame, then the softmax and PV of block ib.
  auto step = [&](int ib, auto bufc, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2],
                  const KeyBlockRec &dc, const KeyBlockRec &dn, const KeyBlockRec &dnn) {
    constexpr int kB = decltype(bufc)::value;
    if (ib + 2 < n_blocks) issue(dnn, false, kB);
    if (ib + 1 < n_blocks) {
      issue(dn, true, 2 + (kB ^ 1));
      set_frame(dn.frame);
    }
    softmax_pv(s_cur, dc, kB, lds + (kB ^ 1) * kTileB, s_nxt);
    if (ib + 1 < n_blocks) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      finish_v(dn, kB ^ 1);
      __syncthreads();
    }
  };

  // the records of blocks ib, ib+1 and ib+2 are in registers at step ib
  KeyBlockRec dc = d0, dn = d1, dnn = n_blocks > 2 ? desc(2) : d1;
  for (int ib = 0; ib < n_blocks; ib += 2) {
    step(ib, std::integral_constant<int, 0>{}, sa, sb, dc, dn, dnn);
    dc = dn;
    dn = dnn;
    dnn = ib + 3 < n_blocks ? desc(ib + 3) : dn;
    if (ib + 1 < n_blocks) {
      step(ib + 1, std::integral_constant<int, 1>{}, sb, sa, dc, dn, dnn);
      dc = dn;
      dn = dnn;
      dnn = ib + 4 < n_blocks ? desc(ib + 4) : dn;
    }
  }

  // ---- epilogue (as in the contiguous kernel) ----
  const float l_row = pair_sum(l_lane);
  if (!valid) return;
  if (it.slot < 0) {
    const float inv = 1.f / l_row;
    __bf16 *op = out + ((int64_t)row * h_q + head) * D + 4 * grp;
#pragma unroll
    for (int d = 0; d < kDB; ++d)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 o;
#pragma unroll
        for (int b = 0; b < 4; ++b) o[b] = (__bf16)(acc[d][4 * a + b] * inv);
        *reinterpret_cast<bf16x4 *>(op + 32 * d + 8 * a) = o;
      }
  } else {
    __bf16 *wo = reinterpret_cast<__bf16 *>(ws_o) + ((int64_t)it.slot * kM + m) * D + 4 * grp;
#pragma unroll
    for (int d = 0; d < kDB; ++d)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 o;
#pragma unroll
        for (int b = 0; b < 4; ++b) o[b] = (__bf16)acc[d][4 * a + b];
        *reinterpret_cast<bf16x4 *>(wo + 32 * d + 8 * a) = o;
      }
    if (grp == 0) {
      ws_ml[((int64_t)it.slot * kM + m) * 2 + 0] = m_run;
      ws_ml[((int64_t)it.slot * kM + m) * 2 + 1] = l_row;
    }
  }
}

template <int D, bool kHalf>
__global__ __launch_bounds__(kBfThreads, 2) void attn_bf16_paged_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ pool_k,
    const __bf16 *__restrict__ pool_v, const __bf16 *__restrict__ k_fresh,
    const __bf16 *__restrict__ v_fresh, __bf16 *__restrict__ out,
    const int32_t *__restrict__ rows, const AttnTile *__restrict__ tiles,
    const AttnItem *__restrict__ items, const KeyBlockRec *__restrict__ recs,
    const float2 *__restrict__ angles, float *__restrict__ ws_o, float *__restrict__ ws_ml,
    int h_q, int h_kv, int tile_rows, float scale_log2, int pool_bytes) {
  attn_bf16_paged_body<D, kHalf>(q, pool_k, pool_v, k_fresh, v_fresh, out, rows, tiles, items,
                                 recs, angles, ws_o, ws_ml, h_q, h_kv, tile_rows, scale_log2,
                                 pool_bytes);
}

// ======================== decode over the shared pool =========================
//
// One decode step: the next token of every request (at position N_b, right after its
// query tokens) attends over all of the request's keys -- its pool chunks (rotated by
// delta_c), its recomputed rows (seams and queries, from the fresh buffer) and itself.
// Decode is bound by HBM, so the work is chunk-major: an item streams one pool chunk
// once and scores it against the queries of every request chunk that reads it, each
// query rotated by -delta of its own use (<q, R(delta) k> = <R(-delta) q, k>), so a
// chunk shared by several requests leaves HBM once per step.  Each (use, kv head)
// writes a partial (m, l, O) for its G query heads; the merge folds in the partial of
// the request's fresh rows and the new token itself.

constexpr int kDecWaves = PIC_DECODE_COLS / 32;  // one 32-column MFMA block per wave
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecKB = PIC_DECODE_BLOCK;
constexpr int kDecStages = 2;  // K + V buffers per workgroup: 32 KiB of LDS at D = 128

// Where the keys of one decode piece (part of an (item, kv head) unit) live.  Pool
// pieces read the chunk through its block table, fresh pieces the request's recomputed
// rows; either way the base address excludes the kv head, which sits in the per-lane
// offsets.
struct DecSrc {
  const char *k, *v;      // pool tensors, or the request's first fresh row
  const int32_t *blocks;  // pool block ids of the chunk (pool pieces)
  int n_tab;              // ids its block-table row lists (pool pieces)
  int t_begin, t_end;     // keys of the piece, relative to the chunk or to the fresh rows
  int n_blocks;           // kDecKB-key blocks
  int item, g, rec_off;
  bool pool;
};

// The grid is resident (at most PIC_DECODE_WG_PER_CU workgroups per CU, each with an
// equal run of key blocks cut into pieces by the planner): a workgroup streams the
// blocks of all its pieces back to back, staging the next block -- possibly the first
// of its next piece -- while the current one is scored, so the HBM stream does not
// drain between pieces.
template <int D, bool kHalf>
__device__ __forceinline__ void dec_attn_body(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ pool_k,
    const __bf16 *__restrict__ pool_v, const int32_t *__restrict__ chunk_block_ptr,
    const int32_t *__restrict__ block_ids, const __bf16 *__restrict__ k_fresh,
    const __bf16 *__restrict__ v_fresh, const DecItem *__restrict__ items,
    const int32_t *__restrict__ uses, const int32_t *__restrict__ segs,
    const int32_t *__restrict__ req_row_ptr, const DecPiece *__restrict__ pieces,
    const int32_t *__restrict__ piece_recs, const int32_t *__restrict__ wg_ptr,
    const float2 *__restrict__ angles, __bf16 *__restrict__ ws_o, float *__restrict__ ws_ml,
    int h_q, int h_kv, float scale_log2, int64_t pool_blocks) {
  constexpr int kRowB = D * 2;
  constexpr int kCPR = D / 8;
  constexpr int kTileB = kDecKB * kRowB;
  constexpr int kRPI = 1024 / kRowB;  // rows per direct load (one wave, 16 B a lane)
  constexpr int kRounds = kDecKB / (kRPI * kDecWaves);
  constexpr int kKS = D / 16;
  constexpr int kDB = D / 32;
  constexpr int kPairs = D / 2;
  constexpr int kT = kDecKB / 32;  // 32-key S^T tiles per block
  static_assert(kDecKB == 32 || kDecKB == 64, "one or two 32-key tiles per block");
  static_assert(kRounds * kRPI * kDecWaves == kDecKB, "direct loads must tile the block");
  static_assert(kPoolBlockRows % kRPI == 0, "one direct load stays inside a pool block");
  static_assert(kDecStages >= 2 && kDecStages <= 4, "vmcnt waits cover up to 3 blocks ahead");
  __shared__ __attribute__((aligned(1024))) char lds[2 * kDecStages * kTileB];  // K..., V...

  const int u_begin = wg_ptr[blockIdx.x], u_end = wg_ptr[blockIdx.x + 1];
  const int group = h_q / h_kv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31;
  const int grp = lane >> 5;
  const int q16 = lane >> 4;
  const int i16 = lane & 15;
  const int tok_bytes = h_kv * kRowB;
  const int64_t blk_bytes = (int64_t)kPoolBlockRows * tok_bytes;

  auto load_src = [&](int pi) {
    DecSrc sr;
    const DecPiece pc = pieces[pi];
    sr.item = pc.item;
    sr.g = pc.g;
    sr.rec_off = pc.rec_off;
    const DecItem it = items[pc.item];
    sr.pool = it.src >= 0;
    sr.t_begin = pc.t_begin;
    sr.t_end = pc.t_end;
    sr.n_blocks = (pc.t_end - pc.t_begin + kDecKB - 1) / kDecKB;
    if (sr.pool) {
      sr.k = reinterpret_cast<const char *>(pool_k);
      sr.v = reinterpret_cast<const char *>(pool_v);
      sr.blocks = block_ids + chunk_block_ptr[it.src];
      sr.n_tab = max(0, chunk_block_ptr[it.src + 1] - chunk_block_ptr[it.src]);
    } else {
      const int64_t row0 = (int64_t)req_row_ptr[-1 - it.src] * tok_bytes;
      sr.k = reinterpret_cast<const char *>(k_fresh) + row0;
      sr.v = reinterpret_cast<const char *>(v_fresh) + row0;
      sr.blocks = nullptr;
      sr.n_tab = 0;
    }
    return sr;
  };

  // per-lane offsets of the next block's loads inside a kRPI-row group: row, kv head,
  // swizzled 16-byte chunk
  int nk[kRounds], nv[kRounds];
  auto set_head = [&](int g) {
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int R = kRPI * (kDecWaves * r + wave) + lane / kCPR;  // row in the block
      const int pch = lane % kCPR;
      nk[r] = (lane / kCPR) * tok_bytes + g * kRowB + 16 * (pch ^ swz_k<kCPR>(R));
      nv[r] = (lane / kCPR) * tok_bytes + g * kRowB + 16 * (pch ^ swz_v<kCPR>(R));
    }
  };
  // Stage block j of sr (K and V) into LDS buffer buf.  Each direct load gets a
  // resource that starts at its first row and ends after the rows that are keys of the
  // unit, so the range check alone zeroes rows past t_end (slack rows of a chunk's last
  // pool block included); the scalar offset stays 0.
  auto issue = [&](const DecSrc &sr, int j, int buf, const int (&ok)[kRounds],
                   const int (&ov)[kRounds]) {
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int t = sr.t_begin + j * kDecKB + kRPI * (kDecWaves * r + wave);  // first row
      int rows = min(max(sr.t_end - t, 0), kRPI);
      int64_t off = 0;
      if (sr.pool) {  // a block id outside the pool reads zeros
        // blocks past the chunk's table row read zeros (never the next row's ids)
        const int bid = rows > 0 && t / kPoolBlockRows < sr.n_tab ? sr.blocks[t / kPoolBlockRows] : -1;
        if (bid < 0 || bid >= pool_blocks)
          rows = 0;
        else
          off = bid * blk_bytes + (int64_t)(t % kPoolBlockRows) * tok_bytes;
      } else {
        off = (int64_t)t * tok_bytes;
      }
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc((void *)(sr.k + off), 0, rows * tok_bytes, 0x00020000);
      const __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc((void *)(sr.v + off), 0, rows * tok_bytes, 0x00020000);
      const int dst = buf * kTileB + (kDecWaves * r + wave) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(lds + dst), 16, ok[r], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(lds + kDecStages * kTileB + dst),
                                               16, ov[r], 0, 0, 0);
    }
  };

  int koff[kKS];
  {
    const int r0 = perm_key(0, n);
    const int f = swz_k<kCPR>(r0);
#pragma unroll
    for (int s = 0; s < kKS; ++s) koff[s] = r0 * kRowB + 16 * ((2 * s + grp) ^ f);
  }
  int voff[kDB];
  {
    const int rr = 8 * (q16 >> 1) + (i16 >> 2);
    const int f = swz_v<kCPR>(rr) >> 2;
#pragma unroll
    for (int d = 0; d < kDB; ++d)
      voff[d] = rr * kRowB + 16 * (4 * (d ^ f) + 2 * (q16 & 1) + ((i16 & 3) >> 1)) +
                8 * (i16 & 1);
  }

  if (u_begin >= u_end) return;
  DecSrc cur = load_src(u_begin);
  DecSrc nxt = cur;  // unit of the next block to stage
  int n_ui = u_begin, n_j = 0;
  set_head(cur.g);
  auto advance = [&]() {  // step (n_ui, n_j) to the next block to stage
    if (++n_j == nxt.n_blocks) {
      n_j = 0;
      if (++n_ui < u_end) {
        nxt = load_src(n_ui);
        set_head(nxt.g);
      }
    }
  };
  // Blocks are numbered in streaming order; block x lives in buffer x % kDecStages.
  // `ahead` counts the staged blocks not yet consumed (the current one included).
  int ahead = 0, stage_buf = 0;
#pragma unroll
  for (int i = 0; i < kDecStages - 1; ++i)
    if (n_ui < u_end) {
      issue(nxt, n_j, stage_buf, nk, nv);
      advance();
      ++ahead;
      stage_buf = stage_buf + 1 == kDecStages ? 0 : stage_buf + 1;
    }
  int buf = 0;

  for (int ui = u_begin; ui < u_end; ++ui) {
    if (ui > u_begin) cur = load_src(ui);
    const DecItem it = items[cur.item];
    const int g = cur.g;
    const bool pool = cur.pool;
    // ---- this lane's query column: (use u, head hh) ----
    const int col = 32 * wave + n;
    const int u = col / group, hh = col - u * group;
    const bool valid = u < it.n_uses;
    const bool active = 32 * wave < it.n_uses * group;  // wave-uniform
    const int use = valid ? uses[it.use_begin + u] : 0;
    const int req = !valid ? 0 : (pool ? segs[8 * use + 5] : -1 - use);
    const int seam = (valid && pool) ? segs[8 * use + 2] : 0;
    const int rec = valid ? piece_recs[cur.rec_off + u] : 0;

    bf16x8 qop[kKS];
    {
      const __bf16 *qp = q + ((int64_t)req * h_q + g * group + hh) * D + 8 * grp;
      bf16x8 qo[kKS];
#pragma unroll
      for (int s = 0; s < kKS; ++s)
        qo[s] = valid ? *reinterpret_cast<const bf16x8 *>(qp + 16 * s) : bf16x8{};
      if (pool && valid) {  // into the chunk's local frame: rotate by -delta of this use
        const float2 *cs = angles + (int64_t)use * kPairs;
        if constexpr (!kHalf) {
#pragma unroll
          for (int s = 0; s < kKS; ++s)
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
              const float2 c = cs[8 * s + 4 * grp + j / 2];
              const float a = (float)qo[s][j], b = (float)qo[s][j + 1];
              qop[s][j] = (__bf16)(a * c.x + b * c.y);
              qop[s][j + 1] = (__bf16)(b * c.x - a * c.y);
            }
        } else {
#pragma unroll
          for (int s = 0; s < kKS / 2; ++s)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float2 c = cs[16 * s + 8 * grp + j];
              const float a = (float)qo[s][j], b = (float)qo[s + kKS / 2][j];
              qop[s][j] = (__bf16)(a * c.x + b * c.y);
              qop[s + kKS / 2][j] = (__bf16)(b * c.x - a * c.y);
            }
        }
      } else {
#pragma unroll
        for (int s = 0; s < kKS; ++s) qop[s] = qo[s];
      }
    }

    f32x16 acc[kDB];
#pragma unroll
    for (int d = 0; d < kDB; ++d)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[d][j] = 0.f;
    float m_run = kNegInf, l_lane = 0.f;

    for (int j = 0; j < cur.n_blocks; ++j) {
      if (n_ui < u_end) {  // stage one more block while this one is scored
        issue(nxt, n_j, stage_buf, nk, nv);
        advance();
        ++ahead;
        stage_buf = stage_buf + 1 == kDecStages ? 0 : stage_buf + 1;
      }
      const int later = ahead - 1;  // blocks staged after this one (their loads may pend)
      if (kDecStages > 3 && later >= 3)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(6 * kRounds) : "memory");
      else if (kDecStages > 2 && later == 2)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * kRounds) : "memory");
      else if (later == 1)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kRounds) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      asm volatile("s_barrier" ::: "memory");
      if (active) {  // a wave whose 32 columns are all past the item's uses only stages
        const char *Kb = lds + buf * kTileB;
        const char *Vb = lds + (kDecStages + buf) * kTileB;
        f32x16 sc[kT];
#pragma unroll
        for (int t = 0; t < kT; ++t) {
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) sc[t][jj] = 0.f;
#pragma unroll
          for (int s = 0; s < kKS; ++s) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(Kb + koff[s] + t * 32 * kRowB);
            sc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[s], sc[t], 0, 0, 0);
          }
        }
        const int t0 = cur.t_begin + j * kDecKB;
        if (t0 < seam || t0 + kDecKB > cur.t_end || !valid) {  // seam rows, rows past the keys
#pragma unroll
          for (int t = 0; t < kT; ++t)
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
              const int tk = t0 + perm_key(t, 8 * (jj >> 2) + 4 * grp + (jj & 3));
              if (tk < seam || tk >= cur.t_end || !valid) sc[t][jj] = kNegInf;
            }
        }
        float mx = kNegInf;
#pragma unroll
        for (int t = 0; t < kT; ++t)
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) mx = fmaxf(mx, sc[t][jj]);
        mx = pair_max(mx) * scale_log2;
        if (mx > m_run) {  // exact running max (decode is bound by HBM, not by this VALU)
          const float alpha = __builtin_amdgcn_exp2f(m_run - mx);
          m_run = mx;
          l_lane *= alpha;
#pragma unroll
          for (int d = 0; d < kDB; ++d) acc[d] *= alpha;
        }
        const float base = m_run == kNegInf ? 0.f : m_run;
        bf16x8 pb[2 * kT];
        const bf16x2v ones = {(__bf16)1.f, (__bf16)1.f};
        float ps = 0.f;
#pragma unroll
        for (int qq = 0; qq < 8 * kT; ++qq) {
          const int t = qq >> 3, jj = 2 * (qq & 7);
          bf16x2v pr;
          pr[0] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[t][jj], scale_log2, -base));
          pr[1] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[t][jj + 1], scale_log2, -base));
          pb[2 * t + (jj >> 3)][jj & 7] = pr[0];
          pb[2 * t + (jj >> 3)][(jj & 7) + 1] = pr[1];
          ps = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ps, false);
        }
        l_lane += ps;
#pragma unroll
        for (int c = 0; c < 2 * kT; ++c)
#pragma unroll
          for (int d = 0; d < kDB; ++d) {
            const char *vr = Vb + voff[d] + c * 16 * kRowB;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)vr);
            const s16x4 hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vr + 4 * kRowB));
            bf16x8 a;
            __builtin_memcpy(&a, &lo, 8);
            __builtin_memcpy(reinterpret_cast<char *>(&a) + 8, &hi, 8);
            acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[c], acc[d], 0, 0, 0);
          }
      }
      asm volatile("s_barrier" ::: "memory");  // buffer buf may be refilled next
      --ahead;
      buf = buf + 1 == kDecStages ? 0 : buf + 1;
    }

    // ---- partial (m, l, O) of this (use, kv head, head) ----
    if (active) {
      const float l_row = pair_sum(l_lane);
      if (valid) {
        const int64_t at = (int64_t)rec * group + hh;
        __bf16 *wo = ws_o + at * D + 4 * grp;
#pragma unroll
        for (int d = 0; d < kDB; ++d)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            bf16x4 o;
#pragma unroll
            for (int b = 0; b < 4; ++b) o[b] = (__bf16)acc[d][4 * a + b];
            *reinterpret_cast<bf16x4 *>(wo + 32 * d + 8 * a) = o;
          }
        if (grp == 0) {
          ws_ml[at * 2 + 0] = m_run;
          ws_ml[at * 2 + 1] = l_row;
        }
      }
    }
  }
}

template <int D, bool kHalf>
__global__ __launch_bounds__(kDecThreads, 2) void dec_attn_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ pool_k,
    const __bf16 *__restrict__ pool_v, const int32_t *__restrict__ chunk_block_ptr,
    const int32_t *__restrict__ block_ids, const __bf16 *__restrict__ k_fresh,
    const __bf16 *__restrict__ v_fresh, const DecItem *__restrict__ items,
    const int32_t *__restrict__ uses, const int32_t *__restrict__ segs,
    const int32_t *__restrict__ req_row_ptr, const DecPiece *__restrict__ pieces,
    const int32_t *__restrict__ piece_recs, const int32_t *__restrict__ wg_ptr,
    const float2 *__restrict__ angles, __bf16 *__restrict__ ws_o, float *__restrict__ ws_ml,
    int h_q, int h_kv, float scale_log2, int64_t pool_blocks) {
  dec_attn_body<D, kHalf>(q, pool_k, pool_v, chunk_block_ptr, block_ids, k_fresh, v_fresh,
                          items, uses, segs, req_row_ptr, pieces, piece_recs, wg_ptr, angles,
                          ws_o, ws_ml, h_q, h_kv, scale_log2, pool_blocks);
}

// One workgroup per (request, query head): groups of D/4 lanes fold disjoint subsets
// of the records of (request, kv head) (online log-sum-exp, 4 dims per lane, two
// records' loads in flight per group), group 0 also the new token (score q . k_new,
// weight v_new); the group results are combined in LDS.
constexpr int kDecMergeThreads = 1024;

template <int D>
__global__ __launch_bounds__(kDecMergeThreads) void dec_merge_kernel(
    __bf16 *__restrict__ out, const __bf16 *__restrict__ q, const __bf16 *__restrict__ k_new,
    const __bf16 *__restrict__ v_new, const int32_t *__restrict__ rec_ptr,
    const __bf16 *__restrict__ ws_o, const float *__restrict__ ws_ml, int h_q, int h_kv,
    float scale_log2) {
  constexpr int kC = D / 4;
  constexpr int kDecMergeGroups = kDecMergeThreads / kC;
  __shared__ float part_m[kDecMergeGroups][kC], part_l[kDecMergeGroups][kC];
  __shared__ f32x4 part_o[kDecMergeGroups][kC];
  const int b = blockIdx.x / h_q, h = blockIdx.x - b * h_q;
  const int group = h_q / h_kv;
  const int g = h / group, hh = h - g * group;
  const int gi = threadIdx.x / kC, c4 = threadIdx.x - gi * kC;
  float mmax = kNegInf, den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  if (gi == 0) {  // the new token: one key at its own position
    const __bf16 *qp = q + ((int64_t)b * h_q + h) * D;
    const __bf16 *kp = k_new + ((int64_t)b * h_kv + g) * D;
    float dot = 0.f;
#pragma unroll 4
    for (int d = 0; d < D; d += 8) {
      const bf16x8 a = *reinterpret_cast<const bf16x8 *>(qp + d);
      const bf16x8 k = *reinterpret_cast<const bf16x8 *>(kp + d);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf((float)a[e], (float)k[e], dot);
    }
    mmax = dot * scale_log2;
    den = 1.f;
    const bf16x4 v = *reinterpret_cast<const bf16x4 *>(v_new + ((int64_t)b * h_kv + g) * D + 4 * c4);
#pragma unroll
    for (int e = 0; e < 4; ++e) num[e] = (float)v[e];
  }
  auto fold = [&](float ms, float ls, const f32x4 &os) {
    if (ms == kNegInf) return;
    if (ms > mmax) {
      const float r = __builtin_amdgcn_exp2f(mmax - ms);  // 0 when mmax is -inf
      den *= r;
      num *= r;
      mmax = ms;
    }
    const float w = __builtin_amdgcn_exp2f(ms - mmax);
    den += w * ls;
    num += w * os;
  };
  // kU records per thread per pass, every load issued before the first fold (a request's
  // records number in the hundreds, so most groups finish in one pass)
  constexpr int kU = 8;
  const int s_end = rec_ptr[b * h_kv + g + 1];
  for (int s0 = rec_ptr[b * h_kv + g] + gi; s0 < s_end; s0 += kU * kDecMergeGroups) {
    float2 ml[kU];
    bf16x4 ob[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int sl = s0 + u * kDecMergeGroups;
      ml[u] = make_float2(kNegInf, 0.f);
      if (sl < s_end) {
        const int64_t a = (int64_t)sl * group + hh;
        ml[u] = *reinterpret_cast<const float2 *>(ws_ml + a * 2);
        ob[u] = *reinterpret_cast<const bf16x4 *>(ws_o + a * D + 4 * c4);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (ml[u].x == kNegInf) continue;
      const f32x4 o = {(float)ob[u][0], (float)ob[u][1], (float)ob[u][2], (float)ob[u][3]};
      fold(ml[u].x, ml[u].y, o);
    }
  }
  part_m[gi][c4] = mmax;
  part_l[gi][c4] = den;
  part_o[gi][c4] = num;
  __syncthreads();
  if (gi != 0) return;
  for (int o = 1; o < kDecMergeGroups; ++o) fold(part_m[o][c4], part_l[o][c4], part_o[o][c4]);
  const float inv = 1.f / den;
  bf16x4 res;
#pragma unroll
  for (int e = 0; e < 4; ++e) res[e] = (__bf16)(num[e] * inv);
  *reinterpret_cast<bf16x4 *>(out + ((int64_t)b * h_q + h) * D + 4 * c4) = res;
}

// ================================ fp32 kernel ==================================

constexpr int kF32Waves = 8;
constexpr int kF32Threads = 64 * kF32Waves;
static_assert(kM == 16 * kF32Waves, "one 16-query MFMA column block per wave");

template <int D>
__global__ __launch_bounds__(kF32Threads) void attn_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ kbuf, const float *__restrict__ vbuf,
    float *__restrict__ out, const int32_t *__restrict__ rows, const AttnTile *__restrict__ tiles,
    const AttnItem *__restrict__ items, float *__restrict__ ws_o, float *__restrict__ ws_ml,
    int h_q, int h_kv, int tile_rows, float scale_log2) {
  constexpr int kKs = D + 4;      // K row stride in LDS (floats)
  constexpr int kVs = kKB + 4;    // V^T row stride in LDS (floats)
  constexpr int kUPR = D / 4;     // 16-byte units per key row
  constexpr int kDB = D / 16;
  constexpr int kQOps = D / 4;
  __shared__ __attribute__((aligned(16))) float ks[kKB * kKs];
  __shared__ __attribute__((aligned(16))) float vt[D * kVs];

  const AttnItem it = items[blockIdx.x];
  const AttnTile tile = tiles[it.tile];
  const int g = it.kv_head;
  const int group = h_q / h_kv;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;

  const int m = 16 * wave + col;
  const int row_local = m % tile_rows;
  const int head = g * group + m / tile_rows;
  const bool valid = row_local < tile.n_rows;
  const int row = tile.row_begin + (valid ? row_local : 0);
  const int pos = valid ? rows[row] : -1;

  float qop[kQOps];
  {
    const float *qp = q + ((int64_t)row * h_q + head) * D;
#pragma unroll
    for (int s = 0; s < kQOps; ++s) qop[s] = valid ? qp[4 * s + grp] : 0.f;
  }
  int pos_min = valid ? pos : 0x7fffffff;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) pos_min = min(pos_min, __shfl_xor(pos_min, o));

  f32x4 acc[kDB];
#pragma unroll
  for (int d = 0; d < kDB; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_lane = 0.f;

  const int key_begin = it.key_begin, key_end = it.key_end, key_last = key_end - 1;
  const int64_t tok_stride = (int64_t)h_kv * D;
  const float *kbase = kbuf + (int64_t)tile.tok_base * tok_stride + (int64_t)g * D;
  const float *vbase = vbuf + (int64_t)tile.tok_base * tok_stride + (int64_t)g * D;

  for (int kb0 = key_begin; kb0 < key_end; kb0 += kKB) {
    __syncthreads();
    for (int u = threadIdx.x; u < kKB * kUPR; u += kF32Threads) {
      const int key = u / kUPR, c = u - key * kUPR;
      const int kk = min(kb0 + key, key_last);
      *reinterpret_cast<f32x4 *>(&ks[key * kKs + 4 * c]) =
          *reinterpret_cast<const f32x4 *>(kbase + (int64_t)kk * tok_stride + 4 * c);
    }
    // V transposed: 4 keys x 4 dims per work item
    for (int u = threadIdx.x; u < (kKB / 4) * kUPR; u += kF32Threads) {
      const int quad = u / kUPR, c = u - quad * kUPR;
      f32x4 e[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = min(kb0 + 4 * quad + r, key_last);
        e[r] = *reinterpret_cast<const f32x4 *>(vbase + (int64_t)kk * tok_stride + 4 * c);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4 *>(&vt[(4 * c + j) * kVs + 4 * quad]) =
            f32x4{e[0][j], e[1][j], e[2][j], e[3][j]};
    }
    __syncthreads();

    f32x4 sc[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      sc[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const float *kr = ks + (16 * sb + col) * kKs + grp;
#pragma unroll
      for (int s = 0; s < kQOps; ++s)
        sc[sb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[4 * s], qop[s], sc[sb], 0, 0, 0);
    }
    if (kb0 + kKB - 1 > min(pos_min, key_last)) {
#pragma unroll
      for (int sb = 0; sb < 4; ++sb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb0 + 16 * sb + 4 * grp + i;
          if (key > pos || key > key_last) sc[sb][i] = kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[sb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const bool none = m_new == kNegInf;
    const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float base = none ? 0.f : m_new;
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[sb][i], scale_log2, -base));
        sc[sb][i] = p;
        psum += p;
      }
    l_lane = l_lane * alpha + psum;
#pragma unroll
    for (int d = 0; d < kDB; ++d) acc[d] *= alpha;
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int d = 0; d < kDB; ++d) {
          const float a = vt[(16 * d + col) * kVs + 16 * sb + 4 * grp + i];
          acc[d] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sc[sb][i], acc[d], 0, 0, 0);
        }
  }

  float l_row = l_lane + __shfl_xor(l_lane, 16);
  l_row += __shfl_xor(l_row, 32);
  if (!valid) return;
  if (it.slot < 0) {
    const float inv = 1.f / l_row;
    float *op = out + ((int64_t)row * h_q + head) * D;
#pragma unroll
    for (int d = 0; d < kDB; ++d) *reinterpret_cast<f32x4 *>(op + 16 * d + 4 * grp) = acc[d] * inv;
  } else {
    float *wo = ws_o + ((int64_t)it.slot * kM + m) * D;
#pragma unroll
    for (int d = 0; d < kDB; ++d) *reinterpret_cast<f32x4 *>(wo + 16 * d + 4 * grp) = acc[d];
    if (grp == 0) {
      ws_ml[((int64_t)it.slot * kM + m) * 2 + 0] = m_run;
      ws_ml[((int64_t)it.slot * kM + m) * 2 + 1] = l_row;
    }
  }
}

// ============================ fp32 kernel, paged pool ===========================
//
// The fp32 path over the shared pool: the same tiles, items and key-block records as the
// bf16 paged kernel, the same tiling and math as the fp32 kernel above.  Here the
// rotation goes on the keys: each staged pool row is rotated by R(delta_c) into the
// global frame while it is written to LDS (fp32, from the per-chunk angle table), so the
// query stays as it is; fresh rows are already global.  Rows past a chunk's end and
// pool blocks outside the pool are staged as zeros without a load (slack slots may hold
// anything), and masked.

template <int D, bool kHalf>
__global__ __launch_bounds__(kF32Threads) void attn_f32_paged_kernel(
    const float *__restrict__ q, const float *__restrict__ pool_k,
    const float *__restrict__ pool_v, const float *__restrict__ k_fresh,
    const float *__restrict__ v_fresh, float *__restrict__ out,
    const int32_t *__restrict__ rows, const AttnTile *__restrict__ tiles,
    const AttnItem *__restrict__ items, const KeyBlockRec *__restrict__ recs,
    const float2 *__restrict__ angles, float *__restrict__ ws_o, float *__restrict__ ws_ml,
    int h_q, int h_kv, int tile_rows, float scale_log2) {
  constexpr int kKs = D + 4;
  constexpr int kVs = kKB + 4;
  constexpr int kUPR = D / 4;
  constexpr int kDB = D / 16;
  constexpr int kQOps = D / 4;
  constexpr int kPairs = D / 2;
  static_assert(kKB == 4 * kPoolBlockRows, "a key block is four pool blocks");
  __shared__ __attribute__((aligned(16))) float ks[kKB * kKs];
  __shared__ __attribute__((aligned(16))) float vt[D * kVs];
  __shared__ int kpos[kKB];

  const AttnItem it = items[blockIdx.x];
  const AttnTile tile = tiles[it.tile];
  const int g = it.kv_head;
  const int group = h_q / h_kv;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int fresh_base = tile.pad0, n_fresh = tile.pad1;

  const int m = 16 * wave + col;
  const int row_local = m % tile_rows;
  const int head = g * group + m / tile_rows;
  const bool valid = row_local < tile.n_rows;
  const int row = tile.row_begin + (valid ? row_local : 0);
  const int pos = valid ? rows[row] : -1;

  float qop[kQOps];
  {
    const float *qp = q + ((int64_t)row * h_q + head) * D;
#pragma unroll
    for (int s = 0; s < kQOps; ++s) qop[s] = valid ? qp[4 * s + grp] : 0.f;
  }
  f32x4 acc[kDB];
#pragma unroll
  for (int d = 0; d < kDB; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_lane = 0.f;

  const int64_t tok = (int64_t)h_kv * D;  // floats per token row
  const int n1 = it.key_end - it.key_begin;
  const int n_blocks = n1 + (it.pad1 - it.pad0);
  // address of key `key` of block dsc (K or V), or null: the row stages as zeros
  auto row_ptr = [&](const KeyBlockRec &dsc, int key, bool is_v) -> const float * {
    if (dsc.frame < 0) {
      const int r = dsc.row + key;
      if (r >= n_fresh) return nullptr;
      return (is_v ? v_fresh : k_fresh) + ((int64_t)(fresh_base + r) * h_kv + g) * D;
    }
    if (key >= (dsc.vis >> 8)) return nullptr;  // past the chunk's end
    const int pl = key / kPoolBlockRows;
    const int o = pl == 0 ? dsc.off[0] : pl == 1 ? dsc.off[1] : pl == 2 ? dsc.off[2] : dsc.off[3];
    if (o < 0) return nullptr;
    return reinterpret_cast<const float *>(reinterpret_cast<const char *>(is_v ? pool_v : pool_k) + o) +
           (int64_t)(key % kPoolBlockRows) * tok + (int64_t)g * D;
  };

  for (int ib = 0; ib < n_blocks; ++ib) {
    const KeyBlockRec dsc = recs[ib < n1 ? it.key_begin + ib : it.pad0 + ib - n1];
    const bool pool = dsc.frame >= 0;
    const float2 *cs = angles + (int64_t)(pool ? dsc.frame : 0) * kPairs;
    __syncthreads();
    if (threadIdx.x < kKB) {
      const int r = dsc.row + threadIdx.x;
      kpos[threadIdx.x] = (!pool && r < n_fresh) ? rows[fresh_base + r] : 0x7fffffff;
    }
    // K, rotated into the global frame for pool rows
    if constexpr (!kHalf) {  // pairs (2i, 2i+1): unit c holds pairs 2c and 2c + 1
      for (int u = threadIdx.x; u < kKB * kUPR; u += kF32Threads) {
        const int key = u / kUPR, c = u - key * kUPR;
        const float *src = row_ptr(dsc, key, false);
        f32x4 x = src ? *reinterpret_cast<const f32x4 *>(src + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
        if (pool) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float2 a = cs[2 * c + h];
            const float x0 = x[2 * h], x1 = x[2 * h + 1];
            x[2 * h] = x0 * a.x - x1 * a.y;
            x[2 * h + 1] = x0 * a.y + x1 * a.x;
          }
        }
        *reinterpret_cast<f32x4 *>(&ks[key * kKs + 4 * c]) = x;
      }
    } else {  // pairs (i, i + D/2): units c and c + D/8 hold pairs 4c .. 4c + 3
      for (int u = threadIdx.x; u < kKB * (kUPR / 2); u += kF32Threads) {
        const int key = u / (kUPR / 2), c = u - key * (kUPR / 2);
        const float *src = row_ptr(dsc, key, false);
        f32x4 x = src ? *reinterpret_cast<const f32x4 *>(src + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 y = src ? *reinterpret_cast<const f32x4 *>(src + D / 2 + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
        if (pool) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float2 a = cs[4 * c + e];
            const float x0 = x[e], y0 = y[e];
            x[e] = x0 * a.x - y0 * a.y;
            y[e] = x0 * a.y + y0 * a.x;
          }
        }
        *reinterpret_cast<f32x4 *>(&ks[key * kKs + 4 * c]) = x;
        *reinterpret_cast<f32x4 *>(&ks[key * kKs + D / 2 + 4 * c]) = y;
      }
    }
    // V transposed: 4 keys x 4 dims per work item
    for (int u = threadIdx.x; u < (kKB / 4) * kUPR; u += kF32Threads) {
      const int quad = u / kUPR, c = u - quad * kUPR;
      f32x4 e[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float *src = row_ptr(dsc, 4 * quad + r, true);
        e[r] = src ? *reinterpret_cast<const f32x4 *>(src + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4 *>(&vt[(4 * c + j) * kVs + 4 * quad]) =
            f32x4{e[0][j], e[1][j], e[2][j], e[3][j]};
    }
    __syncthreads();

    f32x4 sc[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      sc[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const float *kr = ks + (16 * sb + col) * kKs + grp;
#pragma unroll
      for (int s = 0; s < kQOps; ++s)
        sc[sb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[4 * s], qop[s], sc[sb], 0, 0, 0);
    }
    {
      const int s0 = dsc.vis & 255, nv = dsc.vis >> 8;
#pragma unroll
      for (int sb = 0; sb < 4; ++sb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 16 * sb + 4 * grp + i;
          const bool ok = pool ? (key >= s0 && key < nv && dsc.base_pos + key <= pos)
                               : kpos[key] <= pos;
          if (!ok) sc[sb][i] = kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[sb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const bool none = m_new == kNegInf;
    const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float base = none ? 0.f : m_new;
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[sb][i], scale_log2, -base));
        sc[sb][i] = p;
        psum += p;
      }
    l_lane = l_lane * alpha + psum;
#pragma unroll
    for (int d = 0; d < kDB; ++d) acc[d] *= alpha;
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int d = 0; d < kDB; ++d) {
          const float a = vt[(16 * d + col) * kVs + 16 * sb + 4 * grp + i];
          acc[d] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sc[sb][i], acc[d], 0, 0, 0);
        }
  }

  float l_row = l_lane + __shfl_xor(l_lane, 16);
  l_row += __shfl_xor(l_row, 32);
  if (!valid) return;
  if (it.slot < 0) {
    const float inv = 1.f / l_row;
    float *op = out + ((int64_t)row * h_q + head) * D;
#pragma unroll
    for (int d = 0; d < kDB; ++d) *reinterpret_cast<f32x4 *>(op + 16 * d + 4 * grp) = acc[d] * inv;
  } else {
    float *wo = ws_o + ((int64_t)it.slot * kM + m) * D;
#pragma unroll
    for (int d = 0; d < kDB; ++d) *reinterpret_cast<f32x4 *>(wo + 16 * d + 4 * grp) = acc[d];
    if (grp == 0) {
      ws_ml[((int64_t)it.slot * kM + m) * 2 + 0] = m_run;
      ws_ml[((int64_t)it.slot * kM + m) * 2 + 1] = l_row;
    }
  }
}

// ================================ merge ========================================

// Combine the split partials of each (tile, kv head) with their log-sum-exp weights:
// one thread per (merge entry, query vector, 8 output dims: 16-byte partial loads), a
// single pass over the slots with an online maximum.  The bf16 kernels store partial O in bf16 (one rounding
// of an unnormalised sum, which the merge weights by exp(m) and divides by the summed
// l), the fp32 kernel in fp32; both sit at the start of the same fp32-sized region.
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(
    T *__restrict__ out, const AttnTile *__restrict__ tiles, const MergeEntry *__restrict__ merges,
    const float *__restrict__ ws_o, const float *__restrict__ ws_ml, int h_q, int h_kv,
    int tile_rows, int n_merge) {
  constexpr int kV = 8;  // output dims per thread
  constexpr int kC = D / kV;
  typedef __attribute__((__vector_size__(kV * sizeof(float)))) float f32x8;
  const int group = h_q / h_kv;
  const int64_t total = (int64_t)n_merge * kM * kC;
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * 256) {
    const int e = (int)(u / (kM * kC));
    const int rem = (int)(u - (int64_t)e * (kM * kC));
    const int m = rem / kC, c = rem - m * kC;
    const MergeEntry me = merges[e];
    const AttnTile tile = tiles[me.tile];
    const int row_local = m % tile_rows;
    if (row_local >= tile.n_rows) continue;
    const int head = me.kv_head * group + m / tile_rows;
    float mmax = kNegInf, den = 0.f;
    f32x8 num = {};
#pragma unroll 4
    for (int s = 0; s < me.n_slots; ++s) {
      const int64_t at = (int64_t)(me.slot_base + s) * kM + m;
      const float2 ml = *reinterpret_cast<const float2 *>(ws_ml + at * 2);
      f32x8 os;
      if constexpr (std::is_same<T, __bf16>::value) {
        const bf16x8 ob =
            *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const __bf16 *>(ws_o) + at * D + kV * c);
#pragma unroll
        for (int i = 0; i < kV; ++i) os[i] = (float)ob[i];
      } else {
        os = *reinterpret_cast<const f32x8 *>(ws_o + at * D + kV * c);
      }
      const float ms = ml.x, ls = ml.y;
      if (ms == kNegInf) continue;
      if (ms > mmax) {
        const float r = __builtin_amdgcn_exp2f(mmax - ms);  // 0 when mmax is -inf
        den *= r;
        num *= r;
        mmax = ms;
      }
      const float w = __builtin_amdgcn_exp2f(ms - mmax);
      den += w * ls;
      num += w * os;
    }
    const float inv = 1.f / den;
    T *op = out + ((int64_t)(tile.row_begin + row_local) * h_q + head) * D + kV * c;
    if constexpr (std::is_same<T, __bf16>::value) {
      bf16x8 o;
#pragma unroll
      for (int i = 0; i < kV; ++i) o[i] = (__bf16)(num[i] * inv);
      *reinterpret_cast<bf16x8 *>(op) = o;
    } else {
      *reinterpret_cast<f32x8 *>(op) = num * inv;
    }
  }
}

template <typename T, int D>
int launch_attn(const PlanHeader &h, const int32_t *plan_dev, const void *q, const void *k,
                const void *v, void *out, float scale, void *workspace, hipStream_t s) {
  const int32_t *rows = plan_dev + h[PIC_H_O_ROWS];
  const AttnTile *tiles = reinterpret_cast<const AttnTile *>(plan_dev + h[PIC_H_O_ATTN_TILES]);
  const AttnItem *items = reinterpret_cast<const AttnItem *>(plan_dev + h[PIC_H_O_ATTN_ITEMS]);
  const MergeEntry *merges = reinterpret_cast<const MergeEntry *>(plan_dev + h[PIC_H_O_MERGE]);
  float *ws_o = static_cast<float *>(workspace);
  float *ws_ml = ws_o ? ws_o + (int64_t)h[PIC_H_N_PARTIALS] * kM * D : nullptr;
  const float scale_log2 = scale * kLog2e;
  const dim3 grid(h[PIC_H_N_ATTN_ITEMS]);
  if constexpr (std::is_same<T, __bf16>::value) {
    hipLaunchKernelGGL((attn_bf16_kernel<D>), grid, dim3(kBfThreads), 0, s,
                       static_cast<const T *>(q), static_cast<const T *>(k),
                       static_cast<const T *>(v), static_cast<T *>(out), rows, tiles, items,
                       ws_o, ws_ml, h[PIC_H_H_Q], h[PIC_H_H_KV], h[PIC_H_TILE_ROWS], scale_log2);
  } else {
    hipLaunchKernelGGL((attn_f32_kernel<D>), grid, dim3(kF32Threads), 0, s,
                       static_cast<const T *>(q), static_cast<const T *>(k),
                       static_cast<const T *>(v), static_cast<T *>(out), rows, tiles, items,
                       ws_o, ws_ml, h[PIC_H_H_Q], h[PIC_H_H_KV], h[PIC_H_TILE_ROWS], scale_log2);
  }
  PIC_LAUNCH_CHECK();
  if (h[PIC_H_N_MERGE] > 0) {
    const int64_t threads = (int64_t)h[PIC_H_N_MERGE] * kM * (D / 8);
    const unsigned blocks = (unsigned)std::min<int64_t>((threads + 255) / 256, 1 << 20);
    hipLaunchKernelGGL((merge_kernel<T, D>), dim3(blocks), dim3(256), 0, s,
                       static_cast<T *>(out), tiles, merges, ws_o, ws_ml, h[PIC_H_H_Q],
                       h[PIC_H_H_KV], h[PIC_H_TILE_ROWS], h[PIC_H_N_MERGE]);
    PIC_LAUNCH_CHECK();
  }
  return PIC_OK;
}

}  // namespace
}  // namespace pic

namespace pic {
namespace {

// Workspace layout: partial O [slots][kM][D], partial (m, l) [slots][kM][2], then for
// paged plans the angle table [n_chunks][D/2] float2 and the key-block records
// [n_kblocks] (sections 16-byte aligned).
size_t partial_bytes(const PlanHeader &h, int head_dim) {
  return (size_t)h[PIC_H_N_PARTIALS] * kM * ((size_t)head_dim + 2) * sizeof(float);
}
size_t angle_offset(const PlanHeader &h, int head_dim) {
  return (partial_bytes(h, head_dim) + 15) / 16 * 16;
}
size_t keyblock_offset(const PlanHeader &h, int head_dim) {
  return angle_offset(h, head_dim) +
         ((size_t)h[PIC_H_N_CHUNKS] * (head_dim / 2) * sizeof(float2) + 15) / 16 * 16;
}

template <int D, bool kHalf>
int launch_paged(const PlanHeader &h, const int32_t *plan_dev, const void *q, const void *pool_k,
                 const void *pool_v, const int32_t *cbp, const int32_t *bids, const void *kf,
                 const void *vf, void *out, double rope_base, float scale, void *workspace,
                 int64_t pool_blocks, hipStream_t s) {
  const int32_t *rows = plan_dev + h[PIC_H_O_ROWS];
  const AttnTile *tiles = reinterpret_cast<const AttnTile *>(plan_dev + h[PIC_H_O_ATTN_TILES]);
  const AttnItem *items = reinterpret_cast<const AttnItem *>(plan_dev + h[PIC_H_O_ATTN_ITEMS]);
  const MergeEntry *merges = reinterpret_cast<const MergeEntry *>(plan_dev + h[PIC_H_O_MERGE]);
  const int32_t *segs = plan_dev + h[PIC_H_O_SEGS];
  const int4 *kblocks = reinterpret_cast<const int4 *>(plan_dev + h[PIC_H_O_KBLOCKS]);
  char *ws = static_cast<char *>(workspace);
  float *ws_o = reinterpret_cast<float *>(ws);
  float *ws_ml = ws_o + (int64_t)h[PIC_H_N_PARTIALS] * kM * D;
  float2 *angles = reinterpret_cast<float2 *>(ws + angle_offset(h, D));
  KeyBlockRec *recs = reinterpret_cast<KeyBlockRec *>(ws + keyblock_offset(h, D));
  const int n_chunks = h[PIC_H_N_CHUNKS];
  if (n_chunks > 0) {
    const int64_t total = (int64_t)n_chunks * (D / 2);
    const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 65535);
    hipLaunchKernelGGL(paged_angles_kernel, dim3(blocks), dim3(256), 0, s, angles, segs,
                       n_chunks, D / 2, make_theta(D, rope_base));
    PIC_LAUNCH_CHECK();
  }
  const int tok_bytes = h[PIC_H_H_KV] * D * 2;
  const int n_kblocks = h[PIC_H_N_KBLOCKS];
  if (n_kblocks > 0) {
    hipLaunchKernelGGL(paged_blocks_kernel, dim3((n_kblocks + 255) / 256), dim3(256), 0, s,
                       recs, kblocks, segs, cbp, bids, n_kblocks, (int)pool_blocks,
                       kPoolBlockRows * tok_bytes);
    PIC_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL((attn_bf16_paged_kernel<D, kHalf>), dim3(h[PIC_H_N_ATTN_ITEMS]),
                     dim3(kBfThreads), 0, s, static_cast<const __bf16 *>(q),
                     static_cast<const __bf16 *>(pool_k), static_cast<const __bf16 *>(pool_v),
                     static_cast<const __bf16 *>(kf), static_cast<const __bf16 *>(vf),
                     static_cast<__bf16 *>(out), rows, tiles, items, recs, angles, ws_o, ws_ml,
                     h[PIC_H_H_Q], h[PIC_H_H_KV], h[PIC_H_TILE_ROWS], scale * kLog2e,
                     (int)(pool_blocks * kPoolBlockRows * tok_bytes));
  PIC_LAUNCH_CHECK();
  if (h[PIC_H_N_MERGE] > 0) {
    const int64_t threads = (int64_t)h[PIC_H_N_MERGE] * kM * (D / 8);
    const unsigned blocks = (unsigned)std::min<int64_t>((threads + 255) / 256, 1 << 20);
    hipLaunchKernelGGL((merge_kernel<__bf16, D>), dim3(blocks), dim3(256), 0, s,
                       static_cast<__bf16 *>(out), tiles, merges, ws_o, ws_ml, h[PIC_H_H_Q],
                       h[PIC_H_H_KV], h[PIC_H_TILE_ROWS], h[PIC_H_N_MERGE]);
    PIC_LAUNCH_CHECK();
  }
  return PIC_OK;
}

// fp32 over the pool: the same angle table, key-block records (with fp32 row bytes) and
// merge as the bf16 path, and attn_f32_paged_kernel.
template <int D, bool kHalf>
int launch_paged_f32(const PlanHeader &h, const int32_t *plan_dev, const void *q,
                     const void *pool_k, const void *pool_v, const int32_t *cbp,
                     const int32_t *bids, const void *kf, const void *vf, void *out,
                     double rope_base, float scale, void *workspace, int64_t pool_blocks,
                     hipStream_t s) {
  const int32_t *rows = plan_dev + h[PIC_H_O_ROWS];
  const AttnTile *tiles = reinterpret_cast<const AttnTile *>(plan_dev + h[PIC_H_O_ATTN_TILES]);
  const AttnItem *items = reinterpret_cast<const AttnItem *>(plan_dev + h[PIC_H_O_ATTN_ITEMS]);
  const MergeEntry *merges = reinterpret_cast<const MergeEntry *>(plan_dev + h[PIC_H_O_MERGE]);
  const int32_t *segs = plan_dev + h[PIC_H_O_SEGS];
  const int4 *kblocks = reinterpret_cast<const int4 *>(plan_dev + h[PIC_H_O_KBLOCKS]);
  char *ws = static_cast<char *>(workspace);
  float *ws_o = reinterpret_cast<float *>(ws);
  float *ws_ml = ws_o + (int64_t)h[PIC_H_N_PARTIALS] * kM * D;
  float2 *angles = reinterpret_cast<float2 *>(ws + angle_offset(h, D));
  KeyBlockRec *recs = reinterpret_cast<KeyBlockRec *>(ws + keyblock_offset(h, D));
  const int n_chunks = h[PIC_H_N_CHUNKS];
  if (n_chunks > 0) {
    const int64_t total = (int64_t)n_chunks * (D / 2);
    const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 65535);
    hipLaunchKernelGGL(paged_angles_kernel, dim3(blocks), dim3(256), 0, s, angles, segs,
                       n_chunks, D / 2, make_theta(D, rope_base));
    PIC_LAUNCH_CHECK();
  }
  const int tok_bytes = h[PIC_H_H_KV] * D * 4;
  const int n_kblocks = h[PIC_H_N_KBLOCKS];
  if (n_kblocks > 0) {
    hipLaunchKernelGGL(paged_blocks_kernel, dim3((n_kblocks + 255) / 256), dim3(256), 0, s,
                       recs, kblocks, segs, cbp, bids, n_kblocks, (int)pool_blocks,
                       kPoolBlockRows * tok_bytes);
    PIC_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL((attn_f32_paged_kernel<D, kHalf>), dim3(h[PIC_H_N_ATTN_ITEMS]),
                     dim3(kF32Threads), 0, s, static_cast<const float *>(q),
                     static_cast<const float *>(pool_k), static_cast<const float *>(pool_v),
                     static_cast<const float *>(kf), static_cast<const float *>(vf),
                     static_cast<float *>(out), rows, tiles, items, recs, angles, ws_o, ws_ml,
                     h[PIC_H_H_Q], h[PIC_H_H_KV], h[PIC_H_TILE_ROWS], scale * kLog2e);
  PIC_LAUNCH_CHECK();
  if (h[PIC_H_N_MERGE] > 0) {
    const int64_t threads = (int64_t)h[PIC_H_N_MERGE] * kM * (D / 8);
    const unsigned blocks = (unsigned)std::min<int64_t>((threads + 255) / 256, 1 << 20);
    hipLaunchKernelGGL((merge_kernel<float, D>), dim3(blocks), dim3(256), 0, s,
                       static_cast<float *>(out), tiles, merges, ws_o, ws_ml, h[PIC_H_H_Q],
                       h[PIC_H_H_KV], h[PIC_H_TILE_ROWS], h[PIC_H_N_MERGE]);
    PIC_LAUNCH_CHECK();
  }
  return PIC_OK;
}

// Decode workspace: record O [n_dec_recs][G][D] in bf16 (the records are HBM traffic
// of an HBM-bound step; each is one rounding of an unnormalised sum the merge weights
// and renormalises), record (m, l) [..][2] fp32, then the angle table [n_chunks][D/2]
// float2; sections 16-byte aligned.
size_t dec_o_bytes(const PlanHeader &h, int head_dim) {
  return ((size_t)h[PIC_H_N_DEC_RECS] * (h[PIC_H_H_Q] / h[PIC_H_H_KV]) * head_dim * 2 + 15) / 16 * 16;
}
size_t dec_record_bytes(const PlanHeader &h, int head_dim) {
  return dec_o_bytes(h, head_dim) +
         ((size_t)h[PIC_H_N_DEC_RECS] * (h[PIC_H_H_Q] / h[PIC_H_H_KV]) * 2 * sizeof(float) + 15) / 16 * 16;
}

template <int D, bool kHalf>
int launch_decode(const PlanHeader &h, const int32_t *plan_dev, const void *q, const void *k_new,
                  const void *v_new, const void *pool_k, const void *pool_v, const int32_t *cbp,
                  const int32_t *bids, const void *kf, const void *vf, void *out, double rope_base,
                  float scale, void *workspace, int64_t pool_blocks, hipStream_t s) {
  const int32_t *segs = plan_dev + h[PIC_H_O_SEGS];
  const DecItem *items = reinterpret_cast<const DecItem *>(plan_dev + h[PIC_H_O_DEC_ITEMS]);
  const int32_t *uses = plan_dev + h[PIC_H_O_DEC_USES];
  const int32_t *rrp = plan_dev + h[PIC_H_O_REQ_ROW_PTR];
  const DecPiece *pieces = reinterpret_cast<const DecPiece *>(plan_dev + h[PIC_H_O_DEC_PIECES]);
  const int32_t *rec_ptr = plan_dev + h[PIC_H_O_DEC_REC_PTR];
  __bf16 *ws_o = static_cast<__bf16 *>(workspace);
  float *ws_ml = reinterpret_cast<float *>(static_cast<char *>(workspace) + dec_o_bytes(h, D));
  float2 *angles =
      reinterpret_cast<float2 *>(static_cast<char *>(workspace) + dec_record_bytes(h, D));
  const int n_chunks = h[PIC_H_N_CHUNKS];
  if (n_chunks > 0) {
    const int64_t total = (int64_t)n_chunks * (D / 2);
    const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 65535);
    hipLaunchKernelGGL(paged_angles_kernel, dim3(blocks), dim3(256), 0, s, angles, segs,
                       n_chunks, D / 2, make_theta(D, rope_base));
    PIC_LAUNCH_CHECK();
  }
  const float scale_log2 = scale * kLog2e;
  if (h[PIC_H_N_DEC_WG] > 0) {
    hipLaunchKernelGGL((dec_attn_kernel<D, kHalf>), dim3(h[PIC_H_N_DEC_WG]), dim3(kDecThreads),
                       0, s, static_cast<const __bf16 *>(q), static_cast<const __bf16 *>(pool_k),
                       static_cast<const __bf16 *>(pool_v), cbp, bids,
                       static_cast<const __bf16 *>(kf), static_cast<const __bf16 *>(vf), items,
                       uses, segs, rrp, pieces, plan_dev + h[PIC_H_O_DEC_PIECE_RECS],
                       plan_dev + h[PIC_H_O_DEC_WG_PTR], angles, ws_o, ws_ml, h[PIC_H_H_Q],
                       h[PIC_H_H_KV], scale_log2, pool_blocks);
    PIC_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL((dec_merge_kernel<D>), dim3(h[PIC_H_N_REQ] * h[PIC_H_H_Q]),
                     dim3(kDecMergeThreads), 0, s, static_cast<__bf16 *>(out),
                     static_cast<const __bf16 *>(q), static_cast<const __bf16 *>(k_new),
                     static_cast<const __bf16 *>(v_new), rec_ptr, ws_o, ws_ml, h[PIC_H_H_Q],
                     h[PIC_H_H_KV], scale_log2);
  PIC_LAUNCH_CHECK();
  return PIC_OK;
}

}  // namespace
}  // namespace pic

extern "C" size_t pic_decode_workspace_bytes(const int32_t *plan_host, int32_t head_dim) {
  using namespace pic;
  const PlanHeader h{plan_host};
  if (!h.valid() || !h[PIC_H_PAGED] || head_dim <= 0) return 0;
  return dec_record_bytes(h, head_dim) + (size_t)h[PIC_H_N_CHUNKS] * (head_dim / 2) * sizeof(float2);
}

extern "C" int pic_decode_attn_paged(
    const int32_t *plan_host, const int32_t *plan_dev, const void *q_new, const void *k_new,
    const void *v_new, const void *pool_k, const void *pool_v, int64_t pool_blocks,
    int32_t block_size, const int32_t *chunk_block_ptr, int32_t n_pool_chunks,
    const int32_t *block_ids, const void *k_fresh, const void *v_fresh, void *out, int32_t dtype,
    int32_t head_dim, int32_t rope_layout, double rope_base, float scale, void *workspace,
    size_t workspace_bytes, void *stream) {
  using namespace pic;
  const PlanHeader h{plan_host};
  if (!h.valid() || !h[PIC_H_PAGED]) return PIC_EINVAL;
  if (dtype != PIC_BF16 && dtype != PIC_F32) return PIC_EINVAL;
  if (rope_layout != PIC_ROPE_ADJACENT && rope_layout != PIC_ROPE_HALF) return PIC_EINVAL;
  if (!resolve_scale(scale, head_dim) || pool_blocks < 0) return PIC_EINVAL;
  if (!(rope_base > 0.0) || !std::isfinite(rope_base)) return PIC_EINVAL;
  if (dtype != PIC_BF16 || block_size != kPoolBlockRows) return PIC_EUNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PIC_EUNSUPPORTED;
  if (h[PIC_H_H_Q] / h[PIC_H_H_KV] > PIC_DECODE_COLS) return PIC_EUNSUPPORTED;
  const int32_t *segs_h = plan_host + h[PIC_H_O_SEGS];
  for (int32_t c = 0; c < h[PIC_H_N_CHUNKS]; ++c)
    if (segs_h[8 * c + 3] >= n_pool_chunks) return PIC_EINVAL;
  if (h[PIC_H_N_REQ] == 0) return PIC_OK;
  if (!plan_dev || !q_new || !k_new || !v_new || !out || !workspace) return PIC_EINVAL;
  if (h[PIC_H_N_CHUNKS] > 0 && (!pool_k || !pool_v || !chunk_block_ptr || !block_ids))
    return PIC_EINVAL;
  if (h[PIC_H_N_ROWS] > 0 && (!k_fresh || !v_fresh)) return PIC_EINVAL;
  if (workspace_bytes < pic_decode_workspace_bytes(plan_host, head_dim)) return PIC_ENOSPC;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool half = rope_layout == PIC_ROPE_HALF;
#define PIC_DEC(D_, H_)                                                                     \
  return launch_decode<D_, H_>(h, plan_dev, q_new, k_new, v_new, pool_k, pool_v,            \
                               chunk_block_ptr, block_ids, k_fresh, v_fresh, out, rope_base, \
                               scale, workspace, pool_blocks, s)
  if (head_dim == 128) {
    if (half) PIC_DEC(128, true);
    PIC_DEC(128, false);
  }
  if (half) PIC_DEC(64, true);
  PIC_DEC(64, false);
#undef PIC_DEC
}

extern "C" size_t pic_attn_workspace_bytes(const int32_t *plan_host, int32_t head_dim) {
  using namespace pic;
  const PlanHeader h{plan_host};
  if (!h.valid() || head_dim <= 0) return 0;
  if (!h[PIC_H_PAGED]) return partial_bytes(h, head_dim);
  return keyblock_offset(h, head_dim) + (size_t)h[PIC_H_N_KBLOCKS] * sizeof(KeyBlockRec);
}

extern "C" int pic_selective_attn_paged(
    const int32_t *plan_host, const int32_t *plan_dev, const void *q, const void *pool_k,
    const void *pool_v, int64_t pool_blocks, int32_t block_size, const int32_t *chunk_block_ptr,
    int32_t n_pool_chunks, const int32_t *block_ids, const void *k_fresh, const void *v_fresh, void *out, int32_t dtype,
    int32_t head_dim, int32_t rope_layout, double rope_base, float scale, void *workspace,
    size_t workspace_bytes, void *stream) {
  using namespace pic;
  const PlanHeader h{plan_host};
  if (!h.valid() || !h[PIC_H_PAGED]) return PIC_EINVAL;
  if (dtype != PIC_BF16 && dtype != PIC_F32) return PIC_EINVAL;
  if (rope_layout != PIC_ROPE_ADJACENT && rope_layout != PIC_ROPE_HALF) return PIC_EINVAL;
  if (!resolve_scale(scale, head_dim) || pool_blocks < 0) return PIC_EINVAL;
  if (!(rope_base > 0.0) || !std::isfinite(rope_base)) return PIC_EINVAL;
  if (block_size != kPoolBlockRows) return PIC_EUNSUPPORTED;
  if (dtype == PIC_BF16 && head_dim != 64 && head_dim != 128) return PIC_EUNSUPPORTED;
  if (dtype == PIC_F32 && head_dim != 16 && head_dim != 32 && head_dim != 64 && head_dim != 128)
    return PIC_EUNSUPPORTED;
  // 32-bit buffer offsets (past-the-end loads sit at pool_bytes + one block)
  const int64_t tok_bytes = (int64_t)h[PIC_H_H_KV] * head_dim * (int64_t)dtype_size(dtype);
  const int64_t pool_bytes = pool_blocks * kPoolBlockRows * tok_bytes;
  if (pool_bytes > 0x7fff0000LL - kPoolBlockRows * tok_bytes ||
      (int64_t)h[PIC_H_N_ROWS] * tok_bytes > 0x7fff0000LL)
    return PIC_EUNSUPPORTED;
  const int32_t *segs_h = plan_host + h[PIC_H_O_SEGS];
  for (int32_t c = 0; c < h[PIC_H_N_CHUNKS]; ++c)
    if (segs_h[8 * c + 3] >= n_pool_chunks) return PIC_EINVAL;
  if (h[PIC_H_N_ATTN_ITEMS] == 0) return PIC_OK;
  if (!plan_dev || !q || !pool_k || !pool_v || !chunk_block_ptr || !block_ids || !k_fresh ||
      !v_fresh || !out)
    return PIC_EINVAL;
  const size_t need = pic_attn_workspace_bytes(plan_host, head_dim);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return PIC_ENOSPC;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool half = rope_layout == PIC_ROPE_HALF;
  if (dtype == PIC_F32) {
#define PIC_PAGED32(D_)                                                                       \
  return half ? launch_paged_f32<D_, true>(h, plan_dev, q, pool_k, pool_v, chunk_block_ptr,     \
                                           block_ids, k_fresh, v_fresh, out, rope_base, scale,  \
                                           workspace, pool_blocks, s)                           \
              : launch_paged_f32<D_, false>(h, plan_dev, q, pool_k, pool_v, chunk_block_ptr,    \
                                            block_ids, k_fresh, v_fresh, out, rope_base, scale, \
                                            workspace, pool_blocks, s)
    switch (head_dim) {
      case 16: PIC_PAGED32(16);
      case 32: PIC_PAGED32(32);
      case 64: PIC_PAGED32(64);
      default: PIC_PAGED32(128);
    }
#undef PIC_PAGED32
  }
#define PIC_PAGED(D_, H_)                                                                    \
  return launch_paged<D_, H_>(h, plan_dev, q, pool_k, pool_v, chunk_block_ptr, block_ids,     \
                              k_fresh, v_fresh, out, rope_base, scale, workspace,             \
                              pool_blocks, s)
  if (head_dim == 128) {
    if (half) PIC_PAGED(128, true);
    PIC_PAGED(128, false);
  }
  if (half) PIC_PAGED(64, true);
  PIC_PAGED(64, false);
#undef PIC_PAGED
}

extern "C" int pic_selective_attn(const int32_t *plan_host, const int32_t *plan_dev,
                                  const void *q, const void *k, const void *v, void *out,
                                  int32_t dtype, int32_t head_dim, float scale, void *workspace,
                                  size_t workspace_bytes, void *stream) {
  using namespace pic;
  const PlanHeader h{plan_host};
  if (!h.valid() || h[PIC_H_PAGED]) return PIC_EINVAL;
  if (dtype != PIC_BF16 && dtype != PIC_F32) return PIC_EINVAL;
  if (!resolve_scale(scale, head_dim)) return PIC_EINVAL;
  // K/V of one request are addressed with 32-bit byte offsets
  if ((int64_t)h[PIC_H_MAX_TOKENS] * h[PIC_H_H_KV] * head_dim * (int64_t)dtype_size(dtype) >
      0x7fff0000LL)
    return PIC_EUNSUPPORTED;
  if (h[PIC_H_N_ATTN_ITEMS] == 0) return PIC_OK;
  if (!plan_dev || !q || !k || !v || !out) return PIC_EINVAL;
  const size_t need = pic_attn_workspace_bytes(plan_host, head_dim);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return PIC_ENOSPC;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == PIC_BF16) {
    switch (head_dim) {
      case 64: return launch_attn<__bf16, 64>(h, plan_dev, q, k, v, out, scale, workspace, s);
      case 128: return launch_attn<__bf16, 128>(h, plan_dev, q, k, v, out, scale, workspace, s);
      default: return PIC_EUNSUPPORTED;
    }
  }
  switch (head_dim) {
    case 16: return launch_attn<float, 16>(h, plan_dev, q, k, v, out, scale, workspace, s);
    case 32: return launch_attn<float, 32>(h, plan_dev, q, k, v, out, scale, workspace, s);
    case 64: return launch_attn<float, 64>(h, plan_dev, q, k, v, out, scale, workspace, s);
    case 128: return launch_attn<float, 128>(h, plan_dev, q, k, v, out, scale, workspace, s);
    default: return PIC_EUNSUPPORTED;
  }
}

// ===================== selective attention without allocation =====================
//
// For callers that cannot allocate (code under HIP graph capture, tight serving loops):
// the split-KV partials live in a file-scope device array instead of a caller
// workspace.  Each GPU holds its own copy for the life of the process; its address is
// looked up once per device (hipGetSymbolAddress, with that device current) and only
// that address is used from the host.  Every call on a GPU shares the array: calls
// that overlap on one GPU race.  Nothing in it needs clearing: every partial slot a
// merge reads is written by its item in the same call (rows past a tile's end are
// skipped by both, and a slot whose keys were all masked carries m = -inf, which the
// merge skips).

static __device__ __align__(256) unsigned char scratch[PIC_ATTN_SCRATCH_BYTES];

namespace pic {
namespace {

constexpr int kMaxDevices = 64;

// Device address of this GPU's scratch array (nullptr on failure).
void *scratch_ptr(int device) {
  static std::mutex mu;
  static void *ptr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[device] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptr[device] = p;
  }
  return ptr[device];
}

}  // namespace
}  // namespace pic

extern "C" int pic_selective_attn_noalloc(const int32_t *plan_host, const int32_t *plan_dev,
                                          const void *q, const void *k, const void *v, void *out,
                                          int32_t dtype, int32_t head_dim, float scale,
                                          void *stream) {
  using namespace pic;
  const PlanHeader h{plan_host};
  if (!h.valid() || h[PIC_H_PAGED]) return PIC_EINVAL;
  if (dtype != PIC_BF16 && dtype != PIC_F32) return PIC_EINVAL;
  if (!resolve_scale(scale, head_dim)) return PIC_EINVAL;
  // every check of pic_selective_attn, then the scratch bound, before any device call
  if (dtype == PIC_BF16 ? (head_dim != 64 && head_dim != 128)
                        : (head_dim != 16 && head_dim != 32 && head_dim != 64 && head_dim != 128))
    return PIC_EUNSUPPORTED;
  if ((int64_t)h[PIC_H_MAX_TOKENS] * h[PIC_H_H_KV] * head_dim * (int64_t)dtype_size(dtype) >
      0x7fff0000LL)
    return PIC_EUNSUPPORTED;
  if (h[PIC_H_N_ATTN_ITEMS] == 0) return PIC_OK;
  if (!plan_dev || !q || !k || !v || !out) return PIC_EINVAL;
  const size_t need = pic_attn_workspace_bytes(plan_host, head_dim);
  if (need > (size_t)PIC_ATTN_SCRATCH_BYTES) return PIC_ENOSPC;
  void *ws = nullptr;
  if (need > 0) {
    int device = -1;
    if (hipGetDevice(&device) != hipSuccess || device < 0 || device >= kMaxDevices)
      return PIC_EDEVICE;
    ws = scratch_ptr(device);
    if (ws == nullptr) return PIC_EDEVICE;
  }
  return pic_selective_attn(plan_host, plan_dev, q, k, v, out, dtype, head_dim, scale, ws, need,
                            stream);
}
