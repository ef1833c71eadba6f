// One decode step over the shared-chunk pool (pic_decode_attn_paged).
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

#include <algorithm>
#include <cmath>

#include "pic_attn_common.h"

namespace pic {
namespace {

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
  // Pool block ids of block j of sr (pieces start on a block boundary, so pool block p
  // of the block holds rows [t_begin + j * kDecKB + 16 p, ... + 16)); -1 for rows past the
  // piece's keys or past the chunk's table row (never the next row's ids).  They are
  // read one block ahead of the loads that use them, so the scalar-load round trip
  // does not hold back the issue of a block.
  constexpr int kPB = kDecKB / kPoolBlockRows;
  auto fetch_ids = [&](const DecSrc &sr, int j, int (&id)[kPB]) {
#pragma unroll
    for (int p = 0; p < kPB; ++p) {
      const int t = sr.t_begin + j * kDecKB + kPoolBlockRows * p;
      id[p] = sr.pool && t < sr.t_end && t / kPoolBlockRows < sr.n_tab ? sr.blocks[t / kPoolBlockRows] : -1;
    }
  };
  // Stage block j of sr (K and V) into LDS buffer buf.  Each direct load gets a
  // resource that starts at its first row and ends after the rows that are keys of the
  // unit, so the range check alone zeroes rows past t_end (slack rows of a chunk's last
  // pool block included); the scalar offset stays 0.
  auto issue = [&](const DecSrc &sr, int j, int buf, const int (&ok)[kRounds],
                   const int (&ov)[kRounds], const int (&id)[kPB]) {
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int t = sr.t_begin + j * kDecKB + kRPI * (kDecWaves * r + wave);  // first row
      // (wave-uniform; kept in a scalar register so the resource is uniform too)
      int rows = __builtin_amdgcn_readfirstlane(min(max(sr.t_end - t, 0), kRPI));
      int64_t off = 0;
      if (sr.pool) {  // a block id outside the pool reads zeros
        const int bid = rows > 0 ? id[(kRPI * (kDecWaves * r + wave)) / kPoolBlockRows] : -1;
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
  int nid[kPB];  // its pool block ids
  set_head(cur.g);
  fetch_ids(nxt, 0, nid);
  auto advance = [&]() {  // step (n_ui, n_j) to the next block to stage
    if (++n_j == nxt.n_blocks) {
      n_j = 0;
      if (++n_ui < u_end) {
        nxt = load_src(n_ui);
        set_head(nxt.g);
      }
    }
    if (n_ui < u_end) fetch_ids(nxt, n_j, nid);
  };
  // Blocks are numbered in streaming order; block x lives in buffer x % kDecStages.
  // `ahead` counts the staged blocks not yet consumed (the current one included).
  int ahead = 0, stage_buf = 0;
#pragma unroll
  for (int i = 0; i < kDecStages - 1; ++i)
    if (n_ui < u_end) {
      issue(nxt, n_j, stage_buf, nk, nv, nid);
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
        issue(nxt, n_j, stage_buf, nk, nv, nid);
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
// weight v_new); the group results are combined pairwise in LDS.
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
  // the group results combine pairwise in LDS, log2(groups) levels
  part_m[gi][c4] = mmax;
  part_l[gi][c4] = den;
  part_o[gi][c4] = num;
  __syncthreads();
#pragma unroll
  for (int half = kDecMergeGroups / 2; half >= 1; half >>= 1) {
    if (gi < half) {
      fold(part_m[gi + half][c4], part_l[gi + half][c4], part_o[gi + half][c4]);
      part_m[gi][c4] = mmax;
      part_l[gi][c4] = den;
      part_o[gi][c4] = num;
    }
    __syncthreads();
  }
  if (gi != 0) return;
  const float inv = 1.f / den;
  bf16x4 res;
#pragma unroll
  for (int e = 0; e < 4; ++e) res[e] = (__bf16)(num[e] * inv);
  *reinterpret_cast<bf16x4 *>(out + ((int64_t)b * h_q + h) * D + 4 * c4) = res;
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

