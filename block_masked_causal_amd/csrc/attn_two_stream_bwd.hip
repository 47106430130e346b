// Two-stream MARS attention backward (dQ, dK, dV) for gfx950.
//
// The pages train the unchanged model on L_mask + L_AR through the two-stream
// attention (papernotes.org notes on "MARS: Enabling Autoregressive Models
// Multi-Token Generation", key design 2 / 关键设计 2; gist.science explainer,
// section 2B), so the training step needs the gradient of that attention.
// With S = scale Q K^T under the mask M (key design 1, equation M_ij),
// P = softmax_row(S), O = P V and the forward's log-sum-exp per row:
//     P = exp(S - lse),  dV = P^T dO,  dP = dO V^T,
//     dS = P * (dP - D),  D = rowsum(dO * O),
//     dQ = scale dS K,    dK = scale dS^T Q.
// Two kernels (and a reduce):
//  * bwd_dq_kernel: the forward's structure (one wave per 32 query rows, the
//    visible K/V tiles staged in LDS); each wave first forms D of its rows
//    from its dO rows and O (and stores it for the next kernel); P is
//    recomputed from lse, dP^T = V dO^T and dQ^T += K^T dS^T with dS^T fed
//    from registers.
//  * bwd_dkv_kernel: one wave per 32 keys and one query head, two waves per
//    SIMD at d = 128 and three at d = 64; it walks only the query blocks that can see its keys (each key's
//    visible rows are at most two intervals), accumulating dK^T and dV^T in
//    registers over one or more query heads of a GQA group. With a group of
//    one head it writes dK, dV directly; otherwise it writes fp32 partials
//    per workgroup's head set and bwd_dkv_reduce_kernel sums them in head
//    order (no atomics: the result is deterministic).
#include <cmath>
#include <type_traits>

#include "attn_common.hpp"

using namespace mars;

namespace {

struct BwdArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const bf16_t* o;
  const bf16_t* dout;
  const float* lse;  // [b, Hq, 2L], natural log
  float* dsum;       // [b, Hq, 2L] workspace: rowsum(dO * O), from the dQ kernel
  float* dkp;        // [b, 2L, Hq, d] workspace: per-query-head dK (group > 1)
  float* dvp;        // [b, 2L, Hq, d] workspace: per-query-head dV (group > 1)
  bf16_t* dq;
  bf16_t* dk;
  bf16_t* dv;
  int batch, L, B, Hq, Hkv, twoL, group, mask_mode;
  float scale, scale_log2;
  int nqt, gh, nhc, rt, nw;  // dQ kernel split, as in the forward
  int hpw;                   // query heads (of one GQA group) per dK/dV workgroup
};

// ------------------------------------------------------------------ dQ ------
template <int D>
struct DqCfg {
  static constexpr int BN = 64;
  static constexpr int CPR = D / 8;
  static constexpr int TSZ = BN * D;
  static constexpr int NBLK = TSZ / 512;
  static constexpr int BMAX = (NBLK + 3) / 4;
};

// One 64-key tile for one wave of 32 query rows: S^T = K Q^T and
// dP^T = V dO^T (lane (j, hf) holds query row j and 16 keys per 32-key half),
// P^T = exp2(cs S^T - lse2_j), dS^T = P^T (dP^T - D_j), dQ^T += K^T dS^T with
// dS^T as the B operand (K slot (hf, e) of a 16-key chunk is key 4 hf + e or
// 8 + 4 hf + e - 4, the keys the lane holds) and K^T from transposing reads.
// Only the keys whose bit is set in vm[n] count for the 32-key half n (bit t:
// the key t past the lane's first key c0 + 32 n + 4 hf).
template <int D>
__device__ __forceinline__ void dq_tile(const bf16_t* __restrict__ Ks,
                                        const bf16_t* __restrict__ Vs,
                                        const bf16x8 (&qf)[D / 16],
                                        const bf16x8 (&dof)[D / 16], f32x16 (&dq)[D / 32],
                                        float lse2, float dsum, float cs, const uint32_t (&vm)[2],
                                        const int (&kad)[D / 16],
                                        const int (&ktr)[2][D / 32]) {
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const bf16x8 ka = *(const bf16x8*)(Ks + kad[c] + 32 * n * D);
      s = mfma32(ka, qf[c], s);
    }
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const bf16x8 va = *(const bf16x8*)(Vs + kad[c] + 32 * n * D);
      dp = mfma32(va, dof[c], dp);
    }
    // the per-key test only where some lane's keys are not all visible (bits
    // 8 (r / 4) + r % 4 are the ones in use)
    if (__builtin_amdgcn_ballot_w64((vm[n] & 0x0F0F0F0Fu) != 0x0F0F0F0Fu) != 0)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + (r & 3);
        s[r] = (vm[n] >> off) & 1u ? s[r] : -INFINITY;
      }
    bf16x8 ds[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pr = fast_exp2(fmaf(s[r], cs, -lse2));
      ds[r >> 3][r & 7] = (bf16_t)(pr * (dp[r] - dsum));
    }
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const int kc = 2 * n + kh;
        const bf16x4 lo = lds_read_tr(Ks + ktr[0][i] + 16 * kc * D);
        const bf16x4 hi = lds_read_tr(Ks + ktr[1][i] + 16 * kc * D);
        const bf16x8 ka = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        dq[i] = mfma32(ka, ds[kh], dq[i]);
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(512, 2) void bwd_dq_kernel(BwdArgs p) {
  using C = DqCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16_t stage0[2 * C::TSZ];
  __shared__ __attribute__((aligned(16))) bf16_t stage1[2 * C::TSZ];
  const int NT = 64 * p.nw;
  (void)NT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, hf = lane >> 5;

  // (batch, KV head, head chunk, query tile), heaviest tiles first
  const int nkv = p.batch * p.Hkv;
  const int hc = blockIdx.x % p.nhc;
  const int kvg = (blockIdx.x / p.nhc) % nkv;
  const int rank = blockIdx.x / (p.nhc * nkv);
  const int b = kvg / p.Hkv;
  const int kvh = kvg % p.Hkv;
  const int h = kvh * p.group + hc * p.gh + w % p.gh;
  const int bm = 32 * p.rt;
  int qt;
  if (p.mask_mode == 0 && (p.L % bm) == 0) {
    const int nqs = p.L / bm;
    qt = (rank & 1) * nqs + (nqs - 1 - (rank >> 1));
  } else {
    qt = p.nqt - 1 - rank;
  }
  const int a0 = qt * bm;
  const int a_last = min(a0 + bm, p.twoL) - 1;

  int r1_hi, r2_lo, r2_hi, full_below;
  rows_key_ranges(a0, a_last, p.L, p.B, p.mask_mode, r1_hi, r2_lo, r2_hi, full_below);
  const int n1 = (r1_hi + C::BN - 1) / C::BN;
  const int n2 = r2_hi > r2_lo ? (r2_hi - r2_lo + C::BN - 1) / C::BN : 0;
  const int ntiles = n1 + n2;
  const int wa0 = a0 + 32 * (w / p.gh);
  const bool wave_live = wa0 < p.twoL;
  const int wa_last = wave_live ? min(wa0 + 31, p.twoL - 1) : wa0;
  int w1_hi, w2_lo, w2_hi, w_full;
  rows_key_ranges(wa0, wa_last, p.L, p.B, p.mask_mode, w1_hi, w2_lo, w2_hi, w_full);

  const int a = wa0 + j;
  int hi1, lo2, hi2;
  row_intervals(a, p.L, p.B, p.mask_mode, hi1, lo2, hi2);
  const bool row_ok = a < p.twoL;

  const size_t qs = (size_t)p.Hq * D, rs = (size_t)p.Hkv * D;
  const rsrc_t rq = make_rsrc(p.q + (size_t)b * p.twoL * qs + (size_t)h * D,
                              (uint32_t)(((p.twoL - 1) * qs + D) * sizeof(bf16_t)));
  const rsrc_t rdo = make_rsrc(p.dout + (size_t)b * p.twoL * qs + (size_t)h * D,
                               (uint32_t)(((p.twoL - 1) * qs + D) * sizeof(bf16_t)));
  const uint32_t kv_bytes = (uint32_t)(((p.twoL - 1) * rs + D) * sizeof(bf16_t));
  const rsrc_t rk = make_rsrc(p.k + (size_t)b * p.twoL * rs + (size_t)kvh * D, kv_bytes);
  const rsrc_t rv = make_rsrc(p.v + (size_t)b * p.twoL * rs + (size_t)kvh * D, kv_bytes);

  bf16x8 qf[D / 16], dof[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const uint32_t off = (uint32_t)((a * qs + 16 * c + 8 * hf) * sizeof(bf16_t));
    qf[c] = __builtin_bit_cast(bf16x8, buf_load16(rq, off));
    dof[c] = __builtin_bit_cast(bf16x8, buf_load16(rdo, off));
  }
  const size_t rowoff = ((size_t)b * p.Hq + h) * p.twoL;
  const float lse2 = row_ok ? p.lse[rowoff + a] * kLog2e : 0.f;
  // D = rowsum(dO * O) of the lane's row: its 8 chunks of 8 columns, then the
  // other half of the row from the partner lane (rows past 2L read as zeros).
  // Written for the dK/dV kernel, which runs after this one.
  float dpart = 0.f;
  {
    const rsrc_t ro = make_rsrc(p.o + (size_t)b * p.twoL * qs + (size_t)h * D,
                                (uint32_t)(((p.twoL - 1) * qs + D) * sizeof(bf16_t)));
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const uint32_t off = (uint32_t)((a * qs + 16 * c + 8 * hf) * sizeof(bf16_t));
      const bf16x8 ov = __builtin_bit_cast(bf16x8, buf_load16(ro, off));
#pragma unroll
      for (int e = 0; e < 8; ++e) dpart = fmaf((float)dof[c][e], (float)ov[e], dpart);
    }
    dpart += __shfl_xor(dpart, 32);
  }
  const float dsum = row_ok ? dpart : 0.f;
  if (row_ok && hf == 0) p.dsum[rowoff + a] = dsum;

  auto tile_c0 = [&](int it) { return it < n1 ? it * C::BN : r2_lo + (it - n1) * C::BN; };

  // K and V tiles: direct global -> LDS loads, rows XOR-permuted (swz_b) so
  // that both the row reads and the transposing K reads hit all 64 banks
  const int wu = __builtin_amdgcn_readfirstlane(w);
  auto issue_tile = [&](int it, bf16_t* st) {
    const int c0 = tile_c0(it);
#pragma unroll
    for (int i = 0; i < C::BMAX; ++i) {
      const int blk = wu + p.nw * i;
      if (blk < C::NBLK) {
        const int u = blk * 64 + lane;
        const int row = u / C::CPR, slot = u % C::CPR;
        const uint32_t off = (uint32_t)(((c0 + row) * rs) * sizeof(bf16_t)) +
                             16 * (slot ^ swz_b<D>(row));
        lds_load16(rk, st + blk * 512, off);
        lds_load16(rv, st + C::TSZ + blk * 512, off);
      }
    }
  };

  // row reads (K for S^T, V for dP^T): row j (+ 32 n), chunk 2c + hf
  int kad[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) kad[c] = j * D + 8 * ((2 * c + hf) ^ swz_b<D>(j));
  // transposing K reads: 16-lane group g reads keys 4 (g / 2) + lane % 16 / 4
  // (+ 8 e, + 16 kc) at columns 32 i + 16 (g % 2) + 4 (lane % 4)
  int ktr[2][D / 32];
  {
    const int low = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int row = 4 * hf + ((lane & 15) >> 2) + 8 * e;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
        ktr[e][i] = row * D + 8 * ((4 * i + low) ^ swz_b<D>(row)) + 4 * (lane & 1);
    }
  }

  f32x16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dq[i] = f32x16{};

  if (ntiles > 0) issue_tile(0, stage0);
#pragma unroll
  for (int c = 0; c < D / 16; ++c) asm volatile("" ::"v"(qf[c]), "v"(dof[c]));
  __syncthreads();

  auto iteration = [&](int it, auto stage_tag) {
    constexpr int STG = decltype(stage_tag)::value;
    if (it + 1 < ntiles) issue_tile(it + 1, STG == 0 ? stage1 : stage0);
    __builtin_amdgcn_sched_barrier(0);
    const bf16_t* Ks = STG == 0 ? stage0 : stage1;
    const bf16_t* Vs = Ks + C::TSZ;
    const int c0 = tile_c0(it);
    const bool in_r1 = it < n1;
    const int lim_lo = in_r1 ? 0 : r2_lo;
    const int lim_hi = in_r1 ? r1_hi : r2_hi;
    const int t_lo = max(c0, lim_lo), t_hi = min(c0 + C::BN, lim_hi);
    const bool need = wave_live && ((t_lo < w1_hi) | ((t_lo < w2_hi) & (w2_lo < t_hi)));
    if (need) {
      // the lane's visible keys of each 32-key half as a bit mask over the
      // keys past kb = c0 + 32 n + 4 hf, within this tile's range
      uint32_t vm[2];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int kb = c0 + 32 * n + 4 * hf;
        vm[n] = row_bits(lim_lo - kb, min(hi1, lim_hi) - kb) |
                row_bits(max(lo2, lim_lo) - kb, min(hi2, lim_hi) - kb);
      }
      // one code path for every tile (a fully visible one has all bits set): the
      // unmasked and interval-specific copies beside it made the registers spill
      dq_tile<D>(Ks, Vs, qf, dof, dq, lse2, dsum, p.scale_log2, vm, kad, ktr);
    }
    __syncthreads();
  };
  for (int it = 0; it < ntiles; it += 2) {
    iteration(it, std::integral_constant<int, 0>{});
    if (it + 1 < ntiles) iteration(it + 1, std::integral_constant<int, 1>{});
  }

  if (!row_ok) return;
  bf16_t* orow = p.dq + (((size_t)b * p.twoL + a) * p.Hq + h) * D;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 pk = {pack_bf16x2(dq[i][4 * g] * p.scale, dq[i][4 * g + 1] * p.scale),
                  pack_bf16x2(dq[i][4 * g + 2] * p.scale, dq[i][4 * g + 3] * p.scale)};
      *(u32x2*)(orow + 32 * i + 8 * g + 4 * hf) = pk;
    }
  }
}

// ------------------------------------------------------------------ dK, dV --
// Workgroup: NW waves over consecutive keys of one batch and hpw query heads
// of one GQA group; wave w owns the 32 keys k0 + 32 w + j. The K rows of a
// wave's keys sit in registers as B fragments, the workgroup's V rows in LDS.
// For each of its heads in turn, the workgroup walks the 64-row query blocks
// that can see its keys through double-buffered LDS stages holding Q, dO, lse
// and D, and the heads' dK^T and dV^T add up in the same registers. Its dK^T and dV^T accumulators (32 keys x d each,
// d / 2 registers per lane) leave room for two waves per SIMD at d = 128 and
// three at d = 64. At d = 128 a workgroup has 8 waves (256 keys): the stages
// and the V tile then fill one CU's LDS with two waves on every SIMD. At d = 64
// three 4-wave workgroups share a CU (49 KiB of LDS each).
template <int D>
struct DkvCfg {
  static constexpr int QB = 64;                 // query rows per staged block (2 x 32)
  static constexpr int CPR = D / 8;
  static constexpr int QSZ = QB * D;            // Q (or dO) block, elements
  static constexpr int NBLK = QSZ / 512;        // 1 KiB blocks per Q (or dO) block
  static constexpr int NW = D == 128 ? 8 : 4;   // waves per workgroup
  static constexpr int KB = 32 * NW;            // keys per workgroup
  static constexpr int VSZ = KB * D;
  // resident workgroups per CU: LDS-bound at d = 128 (132 KiB); three waves per
  // SIMD at d = 64 (168 registers, 49 KiB of LDS each)
  static constexpr int WG_PER_CU = D == 128 ? 1 : 3;
};

// One 32-row query sub-block for one wave's 32 keys. Only the scores of the
// rows whose bit is set in vm count: bit t is the row t past the lane's first
// row (row offsets 8 (r / 4) + r % 4 of accumulator r). Vs points at the
// wave's own V rows. Read offsets (elements): the row reads of chunk c at
// ro[0] + ((16 c) ^ ro[1]), the transposing reads of column group i, half e,
// at to[e][0] + ((32 i) ^ to[e][1]) (one v_xad_u32 each; the XOR is the
// swz_b permutation of the lane's row).
template <int D>
__device__ __forceinline__ void dkv_block(const bf16_t* __restrict__ Qs,
                                          const bf16_t* __restrict__ Ds,
                                          const float* __restrict__ Ls,
                                          const float* __restrict__ Dl,
                                          const bf16_t* __restrict__ Vs,
                                          const bf16x8 (&kf)[D / 16],
                                          f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32],
                                          float cs, uint32_t vm, const int (&ro)[2],
                                          const int (&to)[2][2], int hf) {
  // S = Q K^T and dP = dO V^T: lane (j, hf) holds key j and query rows
  // 8 (r / 4) + 4 hf + r % 4 of the sub-block
  f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const int ad = ro[0] + ((16 * c) ^ ro[1]);
    s = mfma32(*(const bf16x8*)(Qs + ad), kf[c], s);
  }
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const int ad = ro[0] + ((16 * c) ^ ro[1]);
    dp = mfma32(*(const bf16x8*)(Ds + ad), *(const bf16x8*)(Vs + ad), dp);
  }
  // the per-row test only where some lane's rows are not all visible (bits
  // 8 (r / 4) + r % 4 are the ones in use)
  if (__builtin_amdgcn_ballot_w64((vm & 0x0F0F0F0Fu) != 0x0F0F0F0Fu) != 0)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int off = 8 * (r >> 2) + (r & 3);
      s[r] = (vm >> off) & 1u ? s[r] : -INFINITY;
    }
  // lse2 and D of the lane's 16 rows: 4 runs of 4 consecutive rows
  bf16x8 pp[2], ps[2];
#pragma unroll
  for (int gg = 0; gg < 4; ++gg) {
    const f32x4 l4 = *(const f32x4*)(Ls + 8 * gg + 4 * hf);
    const f32x4 d4 = *(const f32x4*)(Dl + 8 * gg + 4 * hf);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * gg + e;
      const float pr = fast_exp2(fmaf(s[r], cs, -l4[e]));
      pp[r >> 3][r & 7] = (bf16_t)pr;
      ps[r >> 3][r & 7] = (bf16_t)(pr * (dp[r] - d4[e]));
    }
  }
  // dV^T += dO^T P and dK^T += Q^T dS: A from transposing reads of the dO / Q
  // block (rows = query slots of the 16-row chunk kc); B from registers
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    const int t0 = to[0][0] + ((32 * i) ^ to[0][1]);
    const int t1 = to[1][0] + ((32 * i) ^ to[1][1]);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const bf16x4 dlo = lds_read_tr(Ds + t0 + 16 * kc * D);
      const bf16x4 dhi = lds_read_tr(Ds + t1 + 16 * kc * D);
      const bf16x8 da = {dlo[0], dlo[1], dlo[2], dlo[3], dhi[0], dhi[1], dhi[2], dhi[3]};
      dv[i] = mfma32(da, pp[kc], dv[i]);
      const bf16x4 qlo = lds_read_tr(Qs + t0 + 16 * kc * D);
      const bf16x4 qhi = lds_read_tr(Qs + t1 + 16 * kc * D);
      const bf16x8 qa = {qlo[0], qlo[1], qlo[2], qlo[3], qhi[0], qhi[1], qhi[2], qhi[3]};
      dk[i] = mfma32(qa, ps[kc], dk[i]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(64 * DkvCfg<D>::NW, D == 64 ? 3 : 2) void bwd_dkv_kernel(BwdArgs p) {
  using C = DkvCfg<D>;
  constexpr int NW = C::NW;
  // per stage: Q block, dO block, then lse2[QB] and D[QB]
  constexpr int STG_EL = 2 * C::QSZ + 4 * C::QB;  // elements (bf16 units); 2 QB floats
  __shared__ __attribute__((aligned(16))) bf16_t stage0[STG_EL];
  __shared__ __attribute__((aligned(16))) bf16_t stage1[STG_EL];
  __shared__ __attribute__((aligned(16))) bf16_t vtile[C::VSZ];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, hf = lane >> 5;

  // key blocks in increasing order (the clean keys near the start see the
  // most rows), the (batch, query head) pairs of one key block side by side
  const int nsets = (p.group + p.hpw - 1) / p.hpw;  // head sets per KV head
  const int nbh = p.batch * p.Hkv * nsets;
  const int kbi = blockIdx.x / nbh;
  const int bh = blockIdx.x % nbh;
  const int hs = bh % nsets;
  const int kvh = (bh / nsets) % p.Hkv;
  const int b = bh / (nsets * p.Hkv);
  const int hq0 = kvh * p.group + hs * p.hpw;        // first query head
  const int nh = min(p.hpw, p.group - hs * p.hpw);  // query heads, in order
  const int k0 = kbi * C::KB;
  // the lane's key and the query rows that see it
  const int key = k0 + 32 * w + j;
  const bool key_ok = key < p.twoL;
  int lo1, hi1, lo2, hi2;
  key_rows(min(key, p.twoL - 1), p.L, p.B, p.mask_mode, lo1, hi1, lo2, hi2);
  if (!key_ok) {
    hi1 = lo1;
    hi2 = lo2;
  }
  // the workgroup's query rows: the union over its keys, as up to two ranges
  const int klast = min(k0 + C::KB, p.twoL) - 1;
  int qa1, qb1, qa2 = 0, qb2 = 0;
  if (p.mask_mode == 1 || (k0 < p.L && klast >= p.L)) {
    qa1 = k0;
    qb1 = p.twoL;
  } else if (klast < p.L) {
    int x1, x2, y1, y2;
    key_rows(k0, p.L, p.B, 0, qa1, x1, qa2, x2);
    key_rows(klast, p.L, p.B, 0, y1, qb1, y2, qb2);
    qb1 = p.L;
    qb2 = p.twoL;
  } else {
    int x1, x2, y1, y2;
    key_rows(k0, p.L, p.B, 0, qa1, x1, y1, y2);
    key_rows(klast, p.L, p.B, 0, x2, qb1, y1, y2);
  }
  const int fb1 = qa1 / C::QB, lb1 = qb1 > qa1 ? (qb1 - 1) / C::QB : fb1 - 1;
  int fb2 = qb2 > qa2 ? qa2 / C::QB : 0, lb2 = qb2 > qa2 ? (qb2 - 1) / C::QB : -1;
  if (fb2 <= lb1) fb2 = lb1 + 1;  // never the same query block twice
  const int nb1 = lb1 - fb1 + 1;
  const int nb2 = lb2 >= fb2 ? lb2 - fb2 + 1 : 0;
  const int nq = nb1 + nb2;  // query blocks per head
  const int niter = nq * nh;

  const size_t qs = (size_t)p.Hq * D, rs = (size_t)p.Hkv * D;
  const uint32_t q_bytes = (uint32_t)(((p.twoL - 1) * qs + D) * sizeof(bf16_t));
  const bf16_t* qbase = p.q + (size_t)b * p.twoL * qs;
  const bf16_t* dobase = p.dout + (size_t)b * p.twoL * qs;
  const uint32_t kv_bytes = (uint32_t)(((p.twoL - 1) * rs + D) * sizeof(bf16_t));
  const rsrc_t rk = make_rsrc(p.k + (size_t)b * p.twoL * rs + (size_t)kvh * D, kv_bytes);
  const rsrc_t rv = make_rsrc(p.v + (size_t)b * p.twoL * rs + (size_t)kvh * D, kv_bytes);

  // K rows of the lane's keys as B fragments (rows past the end read as
  // zeros); V rows of the workgroup's keys into LDS
  bf16x8 kf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    kf[c] = __builtin_bit_cast(
        bf16x8, buf_load16(rk, (uint32_t)((key * rs + 16 * c + 8 * hf) * sizeof(bf16_t))));
  {
    constexpr int VB = C::VSZ / 512;  // 1 KiB blocks of the V tile
#pragma unroll
    for (int i = 0; i < (VB + NW - 1) / NW; ++i) {
      const int blk = w + NW * i;
      if (blk < VB) {
        const int u = blk * 64 + lane;
        const int row = u / C::CPR, slot = u % C::CPR;
        lds_load16(rv, vtile + blk * 512,
                   (uint32_t)(((k0 + row) * rs) * sizeof(bf16_t)) + 16 * (slot ^ swz_b<D>(row)));
      }
    }
  }

  // iteration it: query block it of the two ranges
  // iteration it: query block it % nq of head hq0 + it / nq (the blocks that
  // see the keys are the same for every head)
  auto block_q0 = [&](int it) {
    const int ib = it % nq;
    return (ib < nb1 ? fb1 + ib : fb2 + (ib - nb1)) * C::QB;
  };
  auto head_of = [&](int it) { return hq0 + it / nq; };
  auto issue_block = [&](int it, bf16_t* st) {
    const int q0 = block_q0(it);
    const int hq = head_of(it);
    const rsrc_t rq = make_rsrc(qbase + (size_t)hq * D, q_bytes);
    const rsrc_t rdo = make_rsrc(dobase + (size_t)hq * D, q_bytes);
    // at d = 128, rebuilt per call for the same reason as the read offsets below
    int ln = lane;
    if constexpr (D == 128) asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < (C::NBLK + NW - 1) / NW; ++i) {
      const int blk = w + NW * i;
      if (blk < C::NBLK) {
        const int u = blk * 64 + ln;
        const int row = u / C::CPR, slot = u % C::CPR;
        const uint32_t off = (uint32_t)(((q0 + row) * qs) * sizeof(bf16_t)) +
                             16 * (slot ^ swz_b<D>(row));
        lds_load16(rq, st + blk * 512, off);
        lds_load16(rdo, st + C::QSZ + blk * 512, off);
      }
    }
  };
  // lse2 and D of a block: loaded into registers by wave 0, stored after compute
  float lval = 0.f, dval = 0.f;
  static_assert(C::QB == 64, "one lse / D value per lane of wave 0");
  auto load_ld = [&](int it) {
    if (w == 0) {
      const int a = block_q0(it) + lane;
      const size_t lrow = ((size_t)b * p.Hq + head_of(it)) * p.twoL;
      lval = a < p.twoL ? p.lse[lrow + a] * kLog2e : 0.f;
      dval = a < p.twoL ? p.dsum[lrow + a] : 0.f;
    }
  };
  auto store_ld = [&](bf16_t* st) {
    if (w == 0) {
      float* L2 = (float*)(st + 2 * C::QSZ);
      L2[lane] = lval;
      L2[C::QB + lane] = dval;
    }
  };

  // read offsets. Row reads of the Q / dO block (and of the wave's V rows,
  // whose row j has the same permutation): row j, chunk (2c + hf) ^ swz_b(j).
  // Transposing reads of Q / dO: 16-lane group g reads rows 4 (g / 2) +
  // lane % 16 / 4 (+ 8 e, + 16 kc) at columns 32 i + 16 (g % 2) + 4 (lane % 4),
  // chunk (4i + low) ^ swz_b(row). Both XORs split into a lane constant added
  // to the chunk index XOR a lane constant (dkv_block).
  int ro[2], to[2][2];
  {
    const int sj = swz_b<D>(j);
    ro[0] = j * D + 8 * (hf ^ (sj & 1));
    ro[1] = 16 * (sj >> 1);
    const int low = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int row = 4 * hf + ((lane & 15) >> 2) + 8 * e;
      const int sr = swz_b<D>(row);
      to[e][0] = row * D + 8 * (low ^ (sr & 3)) + 4 * (lane & 1);
      to[e][1] = 32 * (sr >> 2);
    }
  }
  const bf16_t* vrows = vtile + 32 * w * D;

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  if (niter > 0) {
    issue_block(0, stage0);
    load_ld(0);
    store_ld(stage0);
  }
#pragma unroll
  for (int c = 0; c < D / 16; ++c) asm volatile("" ::"v"(kf[c]));
  __syncthreads();

  auto iteration = [&](int it, auto stage_tag) {
    constexpr int STG = decltype(stage_tag)::value;
    bf16_t* nxt = STG == 0 ? stage1 : stage0;
    if (it + 1 < niter) {
      issue_block(it + 1, nxt);
      load_ld(it + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    const bf16_t* Qs = STG == 0 ? stage0 : stage1;
    const bf16_t* Ds = Qs + C::QSZ;
    const float* Ls = (const float*)(Qs + 2 * C::QSZ);
    // two 32-row sub-blocks of the staged 64 rows
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int q0 = block_q0(it) + 32 * sb;
      // the key's visible rows as a bit mask over the rows past the lane's
      // first row rb = q0 + 4 hf (bit t: row rb + t)
      const int rb = q0 + 4 * hf;
      const uint32_t vm = row_bits(lo1 - rb, hi1 - rb) | row_bits(lo2 - rb, hi2 - rb);
      const bool see = (min(hi1, q0 + 32) > max(lo1, q0)) | (min(hi2, q0 + 32) > max(lo2, q0));
      if (__builtin_amdgcn_ballot_w64(see) != 0) {
        const bf16_t* Qb = Qs + 32 * sb * D;
        const bf16_t* Db = Ds + 32 * sb * D;
        const float* Lb = Ls + 32 * sb;
        const float* Dlb = Ls + C::QB + 32 * sb;
        // One code path serves every sub-block (a fully visible one has all
        // bits set): an unmasked copy beside it in the same loop made the
        // register allocation spill at d = 128 and ran slower at d = 64.
        int rol[2] = {ro[0], ro[1]};
        int tol[2][2] = {{to[0][0], to[0][1]}, {to[1][0], to[1][1]}};
        // At d = 128 the six offset bases pass through an empty asm here, so
        // the 16 read offsets are rebuilt next to their reads in every
        // sub-block instead of being hoisted out of the loop: kept live, they
        // pushed K fragments to scratch, reloaded every sub-block.
        if constexpr (D == 128)
          asm volatile("" : "+v"(rol[0]), "+v"(rol[1]), "+v"(tol[0][0]), "+v"(tol[0][1]),
                       "+v"(tol[1][0]), "+v"(tol[1][1]));
        dkv_block<D>(Qb, Db, Lb, Dlb, vrows, kf, dk, dv, p.scale_log2, vm, rol, tol, hf);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (it + 1 < niter) store_ld(nxt);
    __syncthreads();
  };
  for (int it = 0; it < niter; it += 2) {
    iteration(it, std::integral_constant<int, 0>{});
    if (it + 1 < niter) iteration(it + 1, std::integral_constant<int, 1>{});
  }

  // lane (j, hf) holds dK^T / dV^T rows d = 32 i + 8 (r / 4) + 4 hf + r % 4 of its key
  if (!key_ok) return;
  if (p.group > 1) {
    float* dkr = p.dkp + (((size_t)b * p.twoL + key) * p.Hq + hq0) * D;
    float* dvr = p.dvp + (((size_t)b * p.twoL + key) * p.Hq + hq0) * D;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        *(f32x4*)(dkr + 32 * i + 8 * gg + 4 * hf) =
            f32x4{dk[i][4 * gg] * p.scale, dk[i][4 * gg + 1] * p.scale,
                  dk[i][4 * gg + 2] * p.scale, dk[i][4 * gg + 3] * p.scale};
        *(f32x4*)(dvr + 32 * i + 8 * gg + 4 * hf) =
            f32x4{dv[i][4 * gg], dv[i][4 * gg + 1], dv[i][4 * gg + 2],
                  dv[i][4 * gg + 3]};
      }
    return;
  }
  bf16_t* dkr = p.dk + (((size_t)b * p.twoL + key) * p.Hkv + kvh) * D;
  bf16_t* dvr = p.dv + (((size_t)b * p.twoL + key) * p.Hkv + kvh) * D;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const u32x2 pk = {pack_bf16x2(dk[i][4 * gg] * p.scale, dk[i][4 * gg + 1] * p.scale),
                        pack_bf16x2(dk[i][4 * gg + 2] * p.scale, dk[i][4 * gg + 3] * p.scale)};
      *(u32x2*)(dkr + 32 * i + 8 * gg + 4 * hf) = pk;
      const u32x2 pv = {pack_bf16x2(dv[i][4 * gg], dv[i][4 * gg + 1]),
                        pack_bf16x2(dv[i][4 * gg + 2], dv[i][4 * gg + 3])};
      *(u32x2*)(dvr + 32 * i + 8 * gg + 4 * hf) = pv;
    }
  }
}

// dK, dV of a KV head = the sum of its head sets' partials, in head order (a
// set's partial sits in the slot of its first head). One thread per (batch,
// key, KV head, 8 consecutive columns).
template <int D>
__global__ __launch_bounds__(256) void bwd_dkv_reduce_kernel(BwdArgs p) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t total = (size_t)p.batch * p.twoL * p.Hkv * (D / 8);
  if (t >= total) return;
  const int c8 = (int)(t % (D / 8));
  const size_t bkh = t / (D / 8);  // (b, key, kvh) in [b][2L][Hkv] order
  const int kvh = (int)(bkh % p.Hkv);
  const size_t bk = bkh / p.Hkv;
  const float* kp = p.dkp + (bk * p.Hq + (size_t)kvh * p.group) * D + 8 * c8;
  const float* vp = p.dvp + (bk * p.Hq + (size_t)kvh * p.group) * D + 8 * c8;
  float sk[8], sv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sk[e] = sv[e] = 0.f;
  for (int h = 0; h < p.group; h += p.hpw) {
    const f32x4 k0 = *(const f32x4*)(kp + (size_t)h * D), k1 = *(const f32x4*)(kp + (size_t)h * D + 4);
    const f32x4 v0 = *(const f32x4*)(vp + (size_t)h * D), v1 = *(const f32x4*)(vp + (size_t)h * D + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sk[e] += k0[e];
      sk[4 + e] += k1[e];
      sv[e] += v0[e];
      sv[4 + e] += v1[e];
    }
  }
  const size_t o = bkh * D + 8 * c8;
  *(u32x4*)(p.dk + o) = u32x4{pack_bf16x2(sk[0], sk[1]), pack_bf16x2(sk[2], sk[3]),
                              pack_bf16x2(sk[4], sk[5]), pack_bf16x2(sk[6], sk[7])};
  *(u32x4*)(p.dv + o) = u32x4{pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3]),
                              pack_bf16x2(sv[4], sv[5]), pack_bf16x2(sv[6], sv[7])};
}

// Query heads per dK/dV workgroup. A workgroup runs its heads one after the
// other and sums them in registers: fewer fp32 partials are written and
// reduced, and fewer workgroups pay the K/V load and the partial store. But
// its work grows with them, and the launch ends no sooner than its heaviest
// workgroup (the first keys, seen by about all 2L rows of each head). The
// count is the largest whose heaviest workgroup stays within the mean work
// per resident workgroup slot. Visible pairs per head: L (L + 1) under the
// MARS mask, L (2L + 1) under causal-2L.
template <int D>
int dkv_heads_per_wg(const BwdArgs& a) {
  using C = DkvCfg<D>;
  const int ncu = mars_cu_count();
  if (a.group <= 1 || ncu <= 0) return 1;
  const double L = a.L;
  const double pairs = a.mask_mode == 0 ? L * (L + 1) : L * (2 * L + 1);
  // (64-row query block, key block) steps over all heads, per resident slot
  const double per_slot =
      pairs * a.batch * a.Hq / ((double)C::QB * C::KB) / ((double)ncu * C::WG_PER_CU);
  const double heaviest = std::ceil((double)a.twoL / C::QB);  // steps of one head
  const int h = (int)(per_slot / heaviest);
  return h < 1 ? 1 : h > a.group ? a.group : h;
}

template <int D>
int launch_bwd(BwdArgs a, hipStream_t st) {
  a.gh = D == 64 ? 1 : heads_per_wg(a.group);
  a.nhc = a.group / a.gh;
  a.rt = D == 64 ? 4 : 8 / a.gh;
  a.nw = a.gh * a.rt;
  a.nqt = (a.twoL + 32 * a.rt - 1) / (32 * a.rt);
  const double nq = (double)a.batch * a.Hkv * a.nhc * a.nqt;
  const int nkb = (a.twoL + DkvCfg<D>::KB - 1) / DkvCfg<D>::KB;
  a.hpw = dkv_heads_per_wg<D>(a);
  const double nk = (double)a.batch * a.Hkv * ((a.group + a.hpw - 1) / a.hpw) * nkb;
  if (nq >= 2147483647.0 || nk >= 2147483647.0) return MARS_ERR_SHAPE;
  hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((unsigned)nq), dim3(64 * a.nw), 0, st, a);
  hipLaunchKernelGGL(bwd_dkv_kernel<D>, dim3((unsigned)nk), dim3(64 * DkvCfg<D>::NW), 0, st, a);
  if (a.group > 1) {
    const size_t tot = (size_t)a.batch * a.twoL * a.Hkv * (D / 8);
    hipLaunchKernelGGL(bwd_dkv_reduce_kernel<D>, dim3((unsigned)((tot + 255) / 256)), dim3(256),
                       0, st, a);
  }
  return mars_launch_status();
}

}  // namespace

// Layout: dsum [b, Hq, 2L] fp32, then (when Hq > Hkv) the per-query-head dK
// and dV partials [b, 2L, Hq, d] fp32 each, every part 256-byte aligned.
namespace {
size_t bwd_ws_part(size_t bytes) { return (bytes + 255) & ~(size_t)255; }
}  // namespace

extern "C" size_t mars_attn_two_stream_bwd_workspace_bytes(int32_t batch, int32_t L,
                                                           int32_t n_q_heads, int32_t n_kv_heads,
                                                           int32_t head_dim) {
  if (batch < 1 || L < 1 || n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1 ||
      n_q_heads % n_kv_heads)
    return 0;
  const size_t rows = (size_t)batch * 2 * (size_t)L * n_q_heads;
  size_t n = bwd_ws_part(rows * sizeof(float));
  if (n_q_heads > n_kv_heads) n += 2 * bwd_ws_part(rows * head_dim * sizeof(float));
  return n;
}

extern "C" int mars_attn_two_stream_bwd(const void* q, const void* k, const void* v,
                                        const void* o, const void* d_o, const float* lse,
                                        void* dq, void* dk, void* dv, int32_t batch, int32_t L,
                                        int32_t B, int32_t n_q_heads, int32_t n_kv_heads,
                                        int32_t head_dim, int32_t dtype, float softmax_scale,
                                        int32_t mask_mode, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  MARS_REQUIRE(q && k && v && o && d_o && lse && dq && dk && dv, MARS_ERR_NULL);
  MARS_REQUIRE(dtype == MARS_BF16, MARS_ERR_DTYPE);
  MARS_REQUIRE(head_dim == 64 || head_dim == 128, MARS_ERR_UNSUPPORTED);
  MARS_REQUIRE(batch >= 1 && L >= 1 && B >= 1 && B <= L && L <= (1 << 29), MARS_ERR_SHAPE);
  MARS_REQUIRE(n_q_heads >= 1 && n_kv_heads >= 1 && n_q_heads % n_kv_heads == 0, MARS_ERR_SHAPE);
  MARS_REQUIRE(mask_mode == 0 || mask_mode == 1, MARS_ERR_SHAPE);
  MARS_REQUIRE(mars_aligned16(q) && mars_aligned16(k) && mars_aligned16(v) && mars_aligned16(o) &&
                   mars_aligned16(d_o) && mars_aligned16(lse) && mars_aligned16(dq) &&
                   mars_aligned16(dk) && mars_aligned16(dv) && mars_aligned16(workspace),
               MARS_ERR_ALIGN);
  const int twoL = 2 * L;
  MARS_REQUIRE(((double)twoL + 64) * n_q_heads * head_dim * 4 < 2147483647.0, MARS_ERR_SHAPE);
  const size_t need =
      mars_attn_two_stream_bwd_workspace_bytes(batch, L, n_q_heads, n_kv_heads, head_dim);
  MARS_REQUIRE(workspace && workspace_bytes >= need, MARS_ERR_WORKSPACE);

  BwdArgs a;
  a.q = (const bf16_t*)q;
  a.k = (const bf16_t*)k;
  a.v = (const bf16_t*)v;
  a.o = (const bf16_t*)o;
  a.dout = (const bf16_t*)d_o;
  a.lse = lse;
  const size_t rows = (size_t)batch * twoL * n_q_heads;
  a.dsum = (float*)workspace;
  a.dkp = (float*)((char*)workspace + bwd_ws_part(rows * sizeof(float)));
  a.dvp = (float*)((char*)a.dkp + bwd_ws_part(rows * head_dim * sizeof(float)));
  a.dq = (bf16_t*)dq;
  a.dk = (bf16_t*)dk;
  a.dv = (bf16_t*)dv;
  a.batch = batch;
  a.L = L;
  a.B = B;
  a.Hq = n_q_heads;
  a.Hkv = n_kv_heads;
  a.twoL = twoL;
  a.group = n_q_heads / n_kv_heads;
  a.mask_mode = mask_mode;
  a.scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)head_dim);
  a.scale_log2 = a.scale * kLog2e;
  hipStream_t st = (hipStream_t)stream;
  return head_dim == 64 ? launch_bwd<64>(a, st) : launch_bwd<128>(a, st);
}
