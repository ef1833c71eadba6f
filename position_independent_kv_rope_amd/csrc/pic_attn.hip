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
// bf16 kernel (the hot one): 4 waves x 32 queries (a wave owns a quarter of the tile's
// rows with all their heads, and skips key blocks past its last row),
// v_mfma_f32_32x32x16_bf16 for both products, K/V blocks of 64 keys in LDS (three K
// buffers, two V buffers: 80 KB, two workgroups per CU) staged by direct buffer->LDS
// loads (the buffer range clamps rows past the item's keys to zero), K three blocks
// ahead and V one, so that S^T of block i+1 is computed while block i's softmax runs
// (software pipelining inside each wave) and the wait at the end of a block leaves the
// newest K loads in flight, V read transposed for the PV operand with
// ds_read_b64_tr_b16, row sums taken from the bf16 probabilities with v_dot2_f32_bf16.
// fp32 kernel: 8 waves x 16 queries, v_mfma_f32_16x16x4_f32 (fp32 operands, so fp32
// I/O keeps fp32 accuracy), V staged transposed.
#include "pic_attn_common.h"

namespace pic {
namespace {

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
  // K buffers 0..2, V buffers 3..4
  __shared__ __attribute__((aligned(1024))) char lds[5 * kTileB];

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

  // Query columns.  With G <= 32 query heads per KV head, wave w owns rows
  // [w * 32/G, (w + 1) * 32/G) of the tile with all G heads (column n: row n / G, head
  // n % G), so the rows of one wave are a quarter of the tile's span of positions: fewer
  // key blocks straddle them (masking) and the blocks past its last row are skipped.
  // (G is a power of two dividing 128; with G > 32 a wave takes 32 consecutive
  // head-major columns.)  mcol is the column's index in the split partials, which the
  // merge reads head-major: head * tile_rows + row.
  int row_local, hl;
  if (group <= 32) {
    const int lg = __builtin_ctz(group);
    row_local = (wave << (5 - lg)) + (n >> lg);
    hl = n & (group - 1);
  } else {
    const int m = 32 * wave + n;
    row_local = m % tile_rows;
    hl = m / tile_rows;
  }
  const int mcol = hl * tile_rows + row_local;
  const int head = g * group + hl;
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
  int pos_max = pos;  // -1 for a padding column
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    pos_min = min(pos_min, __shfl_xor(pos_min, o));
    pos_max = max(pos_max, __shfl_xor(pos_max, o));
  }
  pos_min = __builtin_amdgcn_readfirstlane(pos_min);
  pos_max = __builtin_amdgcn_readfirstlane(pos_max);

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
  // LDS: K blocks in buffers 0..2, V blocks in buffers 3..4 (buf counts kTileB units).
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
      voff[d] = 3 * kTileB + rr * kRowB + 16 * (4 * (d ^ f) + 2 * (q16 & 1) + ((i16 & 3) >> 1)) +
                8 * (i16 & 1);  // V buffers start after the three K buffers
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
  auto softmax_pv = [&](f32x16 (&sc)[2], int kb0, int Vb_off, const char *Knext,
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
      const char *vr = lds + voff[o % kDB] + Vb_off + (o / kDB) * 16 * kRowB;
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
  // K blocks rotate through three buffers, V blocks through two: block ib's K lives in
  // K buffer ib % 3, its V in V buffer ib % 2.  K is staged three blocks ahead, so the
  // wait at the end of a block leaves the newest K loads in flight.
  issue(kh, voff_k, key_begin, 0);
  issue(vh, voff_v, key_begin, 3);
  if (n_blocks > 1) issue(kh, voff_k, key_begin + kKB, 1);
  if (n_blocks > 2) {
    issue(kh, voff_k, key_begin + 2 * kKB, 2);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kRounds) : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  f32x16 sa[2], sb[2];
  qk(lds, sa);
  __syncthreads();  // K buffer 0 is refilled next

  // Block ib: S^T(ib) is in registers; stage V(ib+1) and K(ib+3), compute S^T(ib+1),
  // then the softmax and PV of block ib.  KC = ib % 3, VC = ib % 2.
  auto step = [&](int ib, auto kc, auto vc, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2]) {
    constexpr int KC = decltype(kc)::value, VC = decltype(vc)::value;
    const int kb0 = key_begin + ib * kKB;
    if (ib + 1 < n_blocks) issue(vh, voff_v, kb0 + kKB, 3 + (VC ^ 1));
    const bool k3 = ib + 3 < n_blocks;
    if (k3) issue(kh, voff_k, kb0 + 3 * kKB, KC);
    // a block past this wave's last row (and every later one) is masked for all its
    // columns: the wave only stages its share of the loads
    if (kb0 <= pos_max) softmax_pv(s_cur, kb0, VC * kTileB, lds + ((KC + 1) % 3) * kTileB, s_nxt);
    if (ib + 1 < n_blocks) {
      if (k3)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kRounds) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  for (int ib = 0; ib < n_blocks; ib += 6) {
    step(ib, I0{}, I0{}, sa, sb);
    if (ib + 1 < n_blocks) step(ib + 1, I1{}, I1{}, sb, sa);
    if (ib + 2 < n_blocks) step(ib + 2, I2{}, I0{}, sa, sb);
    if (ib + 3 < n_blocks) step(ib + 3, I0{}, I1{}, sb, sa);
    if (ib + 4 < n_blocks) step(ib + 4, I1{}, I0{}, sa, sb);
    if (ib + 5 < n_blocks) step(ib + 5, I2{}, I1{}, sb, sa);
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
    __bf16 *wo = reinterpret_cast<__bf16 *>(ws_o) + ((int64_t)it.slot * kM + mcol) * D + 4 * grp;
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
      ws_ml[((int64_t)it.slot * kM + mcol) * 2 + 0] = m_run;
      ws_ml[((int64_t)it.slot * kM + mcol) * 2 + 1] = l_row;
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

// ================================ fp32 kernel ==================================


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
  return launch_merge<T, D>(h, tiles, merges, out, ws_o, ws_ml, s);
}

}  // namespace
}  // namespace pic

extern "C" size_t pic_attn_workspace_bytes(const int32_t *plan_host, int32_t head_dim) {
  using namespace pic;
  const PlanHeader h{plan_host};
  if (!h.valid() || head_dim <= 0) return 0;
  if (!h[PIC_H_PAGED]) return partial_bytes(h, head_dim);
  return keyblock_offset(h, head_dim) + (size_t)h[PIC_H_N_KBLOCKS] * sizeof(KeyBlockRec);
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
