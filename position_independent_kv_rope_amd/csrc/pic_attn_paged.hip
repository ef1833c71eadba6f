// Selective attention over the shared-chunk pool (pic_selective_attn_paged).
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

#include <algorithm>
#include <cmath>

#include "pic_attn_common.h"

namespace pic {
namespace {

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

  // Query columns as in the contiguous kernel: with G <= 32, wave w owns a quarter of
  // the tile's rows with all G heads; mcol is the head-major column index the merge reads.
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
  const int fresh_base = tile.pad0, n_fresh = tile.pad1;

  // the wave's first position, and its last position and row (-1: no valid column)
  int pos_min = valid ? pos : 0x7fffffff;
  int pos_max = pos, row_max = valid ? row : -1;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    pos_min = min(pos_min, __shfl_xor(pos_min, o));
    pos_max = max(pos_max, __shfl_xor(pos_max, o));
    row_max = max(row_max, __shfl_xor(row_max, o));
  }
  pos_min = __builtin_amdgcn_readfirstlane(pos_min);
  pos_max = __builtin_amdgcn_readfirstlane(pos_max);
  row_max = __builtin_amdgcn_readfirstlane(row_max);

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
  // A block no key of which any column of this wave sees: fresh rows after the wave's
  // last row, or a pool block starting past its last position.  Step ib is skipped
  // (the wave only stages its share of the loads) when block ib and block ib+1 are both
  // unseen; a block that is unseen while the next one is not still runs, on stale
  // scores, and its mask then covers every key (fresh keys after every row of the wave,
  // pool keys past pos_min), so it contributes nothing.
  auto unseen = [&](const KeyBlockRec &d) {
    return d.frame < 0 ? fresh_base + d.row > row_max : d.base_pos > pos_max;
  };
  auto step = [&](int ib, auto bufc, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2],
                  const KeyBlockRec &dc, const KeyBlockRec &dn, const KeyBlockRec &dnn) {
    constexpr int kB = decltype(bufc)::value;
    const bool skip = unseen(dc) && (ib + 1 >= n_blocks || unseen(dn));
    if (ib + 2 < n_blocks) issue(dnn, false, kB);
    if (ib + 1 < n_blocks) {
      issue(dn, true, 2 + (kB ^ 1));
      if (!skip) set_frame(dn.frame);
    }
    if (!skip) softmax_pv(s_cur, dc, kB, lds + (kB ^ 1) * kTileB, s_nxt);
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

}  // namespace
}  // namespace pic

namespace pic {
namespace {

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
  return launch_merge<__bf16, D>(h, tiles, merges, out, ws_o, ws_ml, s);
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
  return launch_merge<float, D>(h, tiles, merges, out, ws_o, ws_ml, s);
}

}  // namespace
}  // namespace pic

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

