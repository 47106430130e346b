// Two-stream MARS attention forward (training form) for gfx950.
//
// The mask is the 2L x 2L matrix M of the papernotes.org notes on "MARS:
// Enabling Autoregressive Models Multi-Token Generation", key design 1
// (关键设计 1), equation M_ij, over z = [x; x~] with beta(t) = ceil(t/B).
// It is never materialised: every query row a owns at most two visible key
// intervals, computed once per row in registers,
//     clean row a < L : [0, a]
//     mask row a >= L : [0, b*B) and [L + b*B, a]      (t = a - L, b = t / B)
// and a key c is visible iff it lies in one of them. Whole key tiles outside
// a query tile's intervals are never loaded, and tiles entirely inside them
// skip the per-element test.
#include "mars_common.hpp"

using namespace mars;

namespace {

struct TwoStreamArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int batch, L, B, Hq, Hkv, twoL, group;
  float scale_log2;  // softmax_scale * log2(e): scores are kept in log2 units
  int mask_mode;     // 0 = MARS two-stream mask, 1 = causal over all 2L
  int nqt;           // query tiles per (batch, head)
  int gh, nhc, rt, nw;  // bf16 path: heads per workgroup, head chunks per group,
                        // 32-row tiles per workgroup, waves per workgroup
};

// Visible keys of row a: c < hi1, or lo2 <= c < hi2.
__device__ __forceinline__ void row_intervals(int a, int L, int B, int mode, int& hi1, int& lo2,
                                              int& hi2) {
  if (mode == 1 || a < L) {
    hi1 = a + 1;
    lo2 = 0;
    hi2 = 0;
    return;
  }
  const int bb = ((a - L) / B) * B;
  hi1 = bb;
  lo2 = L + bb;
  hi2 = a + 1;
}

__device__ __forceinline__ bool in_rows(int c, int hi1, int lo2, int hi2) {
  return (c < hi1) | ((c >= lo2) & (c < hi2));
}

// ---------------------------------------------------------------------------
// float32 path: one wave per 64 query rows, K/V staged in LDS 32 keys at a
// time, one query row per lane. Used for the small fp32 configuration.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void two_stream_f32_kernel(TwoStreamArgs p) {
  constexpr int KT = 32;
  __shared__ float Ks[KT][D];
  __shared__ float Vs[KT][D];
  const int lane = threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int a = blockIdx.x * 64 + lane;
  const int kvh = h / p.group;
  const bool valid = a < p.twoL;
  const float* Q = (const float*)p.q;
  const float* K = (const float*)p.k;
  const float* V = (const float*)p.v;
  const size_t qrow = ((size_t)b * p.twoL + (valid ? a : 0)) * p.Hq + h;

  float q[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = valid ? Q[qrow * D + d] * p.scale_log2 : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  int hi1, lo2, hi2;
  row_intervals(a, p.L, p.B, p.mask_mode, hi1, lo2, hi2);
  const int a_last = min((int)blockIdx.x * 64 + 63, p.twoL - 1);
  for (int c0 = 0; c0 <= a_last; c0 += KT) {
    __syncthreads();
    for (int idx = lane; idx < KT * D; idx += 64) {
      const int c = c0 + idx / D, d = idx % D;
      const size_t kr = ((size_t)b * p.twoL + c) * p.Hkv + kvh;
      Ks[idx / D][d] = c < p.twoL ? K[kr * D + d] : 0.f;
      Vs[idx / D][d] = c < p.twoL ? V[kr * D + d] : 0.f;
    }
    __syncthreads();
    for (int jj = 0; jj < KT; ++jj) {
      const int c = c0 + jj;
      if (!valid || c >= p.twoL || !in_rows(c, hi1, lo2, hi2)) continue;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(q[d], Ks[jj][d], s);
      const float mn = fmaxf(m, s);
      const float alpha = exp2f(m - mn);
      const float pe = exp2f(s - mn);
      l = l * alpha + pe;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(o[d], alpha, pe * Vs[jj][d]);
      m = mn;
    }
  }
  if (!valid) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* O = (float*)p.o;
#pragma unroll
  for (int d = 0; d < D; ++d) O[qrow * D + d] = o[d] * inv;
  if (p.lse) p.lse[((size_t)b * p.Hq + h) * p.twoL + a] = (m + log2f(l)) * kLn2;
}

// ---------------------------------------------------------------------------
// bfloat16 MFMA path.
//
// Workgroup = 4 waves = 128 query rows of one (batch, q-head); each wave owns
// 32 rows. Scores are computed transposed, S^T = K Q^T, with the 32x32x16
// MFMA: lane (j = l % 32, hf = l / 32) then holds query row j and 16 of the
// keys of each 32-key sub-tile, so the row softmax needs one cross-lane
// exchange (lane l <-> l ^ 32). The probabilities stay in registers and feed
// O^T = V^T P^T directly as the B operand: K slot (hf, e) of a 16-key chunk
// is mapped to key 4*hf + e (e < 4) or 8 + 4*hf + e - 4 (e >= 4), exactly the
// keys the lane already holds. V is written to LDS transposed ([d][key]) so
// that the A operand is two 8-byte LDS reads.
// ---------------------------------------------------------------------------
template <int D>
struct Cfg {
  static constexpr int BN = 64;       // keys per tile
  static constexpr int KST = D + 8;   // K tile row stride in LDS (elements)
  static constexpr int VST = BN + 4;  // V^T tile row stride in LDS (elements)
  static constexpr int KSZ = BN * KST;
  static constexpr int VSZ = D * VST;
  static constexpr int KLOADS = BN * D / 8 / 256;             // 16-byte K loads per thread
  static constexpr int VPATCH = (BN / 4) * (D / 8);           // 4-key x 8-dim V patches
  static constexpr int VLOADS = (VPATCH + 255) / 256;         // patches per thread
  static constexpr size_t LDS_BYTES = 2 * (KSZ + VSZ) * sizeof(bf16_t);
};

// V^T tiles are stored in groups of 4 keys (8 bytes); group cg of row `row`
// sits at group position cg ^ vt_swizzle(row). Writers cover rows 8 apart and
// readers 16 consecutive rows per LDS cycle; this XOR keeps both on distinct
// banks (the unswizzled write pattern hit the same 2 of 32 banks).
__device__ __forceinline__ int vt_swizzle(int row) { return (row >> 4) & 15; }

// Rescaling of the running output is deferred until a row maximum grows by
// more than 2^8: until then exp2(s - m) stays below 256, which neither fp32
// nor bf16 minds, and the final O / l is unchanged by which m was used.
constexpr float kLazyRescale = 8.0f;

constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, one L2 each

// One 64-key tile for one wave (32 query rows): S^T = K Q^T, online softmax,
// O^T += V^T P^T. MASKED applies the per-element visibility test; unmasked
// tiles are fully visible to every row of the wave.
// Lane (j, hf) holds keys kb + 32n + 8(r/4) + (r%4) of its row, kb = c0 + 4hf.
template <int D, bool MASKED>
__device__ __forceinline__ void tile_step(const bf16_t* __restrict__ Ks,
                                          const bf16_t* __restrict__ Vt,
                                          const bf16x8 (&qf)[D / 16], f32x16 (&o)[D / 32],
                                          float& m, float& l, float cs, int kb, int lo_a,
                                          int hi_a, int lo_b, int hi_b, int j, int hf) {
  using C = Cfg<D>;
  f32x16 s[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    s[n] = f32x16{};
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const bf16x8 ka = *(const bf16x8*)(Ks + (32 * n + j) * C::KST + 16 * c + 8 * hf);
      s[n] = mfma32(ka, qf[c], s[n]);
    }
  }
  if (MASKED) {
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = kb + 32 * n + 8 * (r >> 2) + (r & 3);
        const bool vis = ((c >= lo_a) & (c < hi_a)) | ((c >= lo_b) & (c < hi_b));
        s[n][r] = vis ? s[n][r] : -INFINITY;
      }
  }
  // row max of the raw scores (the scale is positive, so it commutes with max)
  float mt = -INFINITY;
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[n][r]);
  mt = fmaxf(mt, __shfl_xor(mt, 32)) * cs;
  const bool grow = mt > m + kLazyRescale;
  if (__ballot(grow)) {
    const float mnew = grow ? mt : m;
    // 1 when unchanged (also when still -inf), 0 when the first key arrives
    const float alpha = m == mnew ? 1.f : fast_exp2(m - mnew);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) o[i] *= alpha;
    m = mnew;
  }
  const float nm = m == -INFINITY ? 0.f : -m;
  float rsum = 0.f;
  bf16x8 pb[4];
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(fmaf(s[n][r], cs, nm));
      rsum += e;
      pb[2 * n + (r >> 3)][r & 7] = (bf16_t)e;
    }
  l += rsum;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    const int row = 32 * i + j;
    const bf16_t* vrow = Vt + row * C::VST;
    const int sw = vt_swizzle(row);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const bf16x4 vlo = *(const bf16x4*)(vrow + 4 * ((4 * kc + hf) ^ sw));
      const bf16x4 vhi = *(const bf16x4*)(vrow + 4 * ((4 * kc + 2 + hf) ^ sw));
      const bf16x8 va = {vlo[0], vlo[1], vlo[2], vlo[3], vhi[0], vhi[1], vhi[2], vhi[3]};
      o[i] = mfma32(va, pb[kc], o[i]);
    }
  }
}

// Key ranges a block of query rows [a0, a_last] needs: r1 = [0, r1_hi) and
// r2 = [r2_lo, r2_hi); keys below full_below are visible to every row.
__device__ __forceinline__ void rows_key_ranges(int a0, int a_last, int L, int B, int mode,
                                                int& r1_hi, int& r2_lo, int& r2_hi,
                                                int& full_below) {
  r2_lo = 0;
  r2_hi = 0;
  if (mode == 1 || a_last < L) {
    r1_hi = a_last + 1;
    full_below = a0 + 1;          // causal: fully visible iff every key <= a0
  } else if (a0 >= L) {
    const int t0 = a0 - L, t1 = a_last - L;
    r1_hi = (t1 / B) * B;         // clean keys of strictly earlier blocks
    full_below = (t0 / B) * B;
    r2_lo = L + full_below;       // mask keys of the blocks these rows sit in
    r2_hi = a_last + 1;
  } else {
    r1_hi = a_last + 1;           // rows straddle the stream boundary: test every key
    full_below = 0;
  }
}

// Workgroup = nw waves, each owning one (query head, 32-row tile). The heads
// of one GQA group that share a K/V head sit side by side (gh heads x rt row
// tiles = nw), so every K/V tile staged through LDS feeds 32 * nw query rows.
template <int D>
__global__ __launch_bounds__(512, 2) void two_stream_bf16_kernel(TwoStreamArgs p) {
  using C = Cfg<D>;
  extern __shared__ __attribute__((aligned(16))) bf16_t lds[];
  const int NT = 64 * p.nw;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int j = lane & 31, hf = lane >> 5;

  // ---- which (batch, KV head, head chunk, query tile) ---------------------
  // Workgroups are dealt to the 8 XCDs round-robin (block i runs on XCD i % 8).
  // When the (batch, KV head) streams split evenly over the XCDs, each XCD owns
  // whole streams, so every query head reading one K/V stream meets it in one
  // L2. Within an XCD the streams run one after another, heaviest query tiles
  // first, with the head chunks of one query tile dispatched side by side.
  const int nkv = p.batch * p.Hkv;
  int kvg, hc, rank;
  if (nkv % kXcds == 0) {
    const int k = blockIdx.x / kXcds;
    const int per_stream = p.nhc * p.nqt;
    kvg = blockIdx.x % kXcds + kXcds * (k / per_stream);
    rank = (k % per_stream) / p.nhc;
    hc = k % p.nhc;
  } else {
    hc = blockIdx.x % p.nhc;
    kvg = (blockIdx.x / p.nhc) % nkv;
    rank = blockIdx.x / (p.nhc * nkv);
  }
  const int b = kvg / p.Hkv;
  const int kvh = kvg % p.Hkv;
  const int h = kvh * p.group + hc * p.gh + w % p.gh;
  const int bm = 32 * p.rt;
  int qt;
  if (p.mask_mode == 0 && (p.L % bm) == 0) {
    const int nqs = p.L / bm;  // tiles per stream; clean tile i and mask tile i cost alike
    qt = (rank & 1) * nqs + (nqs - 1 - (rank >> 1));
  } else {
    qt = p.nqt - 1 - rank;
  }
  const int a0 = qt * bm;
  const int a_last = min(a0 + bm, p.twoL) - 1;

  // key ranges of the whole workgroup (what gets staged) and of this wave
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

  // ---- this lane's query row and its visible key intervals ---------------
  const int a = wa0 + j;
  int hi1, lo2, hi2;
  row_intervals(a, p.L, p.B, p.mask_mode, hi1, lo2, hi2);

  // buffer views: reads past the end of this (batch, head) slice return 0
  const size_t qs = (size_t)p.Hq * D, rs = (size_t)p.Hkv * D;
  const rsrc_t rq = make_rsrc((const bf16_t*)p.q + (size_t)b * p.twoL * qs + (size_t)h * D,
                              (uint32_t)(((p.twoL - 1) * qs + D) * sizeof(bf16_t)));
  const uint32_t kv_bytes = (uint32_t)(((p.twoL - 1) * rs + D) * sizeof(bf16_t));
  const rsrc_t rk = make_rsrc((const bf16_t*)p.k + (size_t)b * p.twoL * rs + (size_t)kvh * D,
                              kv_bytes);
  const rsrc_t rv = make_rsrc((const bf16_t*)p.v + (size_t)b * p.twoL * rs + (size_t)kvh * D,
                              kv_bytes);

  bf16x8 qf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    qf[c] = __builtin_bit_cast(
        bf16x8, buf_load16(rq, (uint32_t)((a * qs + 16 * c + 8 * hf) * sizeof(bf16_t))));

  constexpr int KCH = C::BN * D / 8;                   // 16-byte chunks per K tile
  constexpr int KMAX = (KCH + 5 * 64 - 1) / (5 * 64);  // per thread, at >= 5 waves
  constexpr int VMAX = (C::VPATCH + 5 * 64 - 1) / (5 * 64);
  u32x4 kreg[KMAX];
  u32x4 vreg[VMAX][4];

  auto tile_c0 = [&](int it) { return it < n1 ? it * C::BN : r2_lo + (it - n1) * C::BN; };

  auto load_tile = [&](int it) {
    const int c0 = tile_c0(it);
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      const int idx = min(tid + NT * i, KCH - 1);
      const int row = idx / (D / 8), ch = idx % (D / 8);
      kreg[i] = buf_load16(rk, (uint32_t)(((c0 + row) * rs + ch * 8) * sizeof(bf16_t)));
    }
#pragma unroll
    for (int i = 0; i < VMAX; ++i) {
      const int pi = min(tid + NT * i, C::VPATCH - 1);
      const int dg = pi % (D / 8), kg = pi / (D / 8);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        vreg[i][rr] =
            buf_load16(rv, (uint32_t)(((c0 + 4 * kg + rr) * rs + dg * 8) * sizeof(bf16_t)));
    }
  };

  auto store_tile = [&](int buf) {
    bf16_t* Ks = lds + buf * (C::KSZ + C::VSZ);
    bf16_t* Vt = Ks + C::KSZ;
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      const int idx = tid + NT * i;
      if (idx < KCH) {
        const int row = idx / (D / 8), ch = idx % (D / 8);
        *(u32x4*)(Ks + row * C::KST + ch * 8) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VMAX; ++i) {
      const int pi = tid + NT * i;
      if (pi >= C::VPATCH) continue;
      const int dg = pi % (D / 8), kg = pi / (D / 8);
#pragma unroll
      for (int dw = 0; dw < 4; ++dw) {
        const uint32_t x0 = vreg[i][0][dw], x1 = vreg[i][1][dw];
        const uint32_t x2 = vreg[i][2][dw], x3 = vreg[i][3][dw];
        // dimension 8*dg + 2*dw: low halves; dimension 8*dg + 2*dw + 1: high halves
        // byte permutes: lo = {x0.lo16, x1.lo16}, hi = {x0.hi16, x1.hi16}
        u32x2 lo = {__builtin_amdgcn_perm(x1, x0, 0x05040100u),
                    __builtin_amdgcn_perm(x3, x2, 0x05040100u)};
        u32x2 hi = {__builtin_amdgcn_perm(x1, x0, 0x07060302u),
                    __builtin_amdgcn_perm(x3, x2, 0x07060302u)};
        const int r0 = 8 * dg + 2 * dw, r1 = r0 + 1;
        *(u32x2*)(Vt + r0 * C::VST + 4 * (kg ^ vt_swizzle(r0))) = lo;
        *(u32x2*)(Vt + r1 * C::VST + 4 * (kg ^ vt_swizzle(r1))) = hi;
      }
    }
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  float m = -INFINITY, l = 0.f;

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  // The query fragments must have landed before the loop: otherwise the
  // wait-count bookkeeping treats them as in flight on every iteration and
  // each tile would stall on its own prefetch.
#pragma unroll
  for (int c = 0; c < D / 16; ++c) asm volatile("" ::"v"(qf[c]));
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    if (it + 1 < ntiles) load_tile(it + 1);
    // keep the prefetch issued before the compute, and its LDS stores after it
    __builtin_amdgcn_sched_barrier(0);

    const bf16_t* Ks = lds + (it & 1) * (C::KSZ + C::VSZ);
    const bf16_t* Vt = Ks + C::KSZ;
    const int c0 = tile_c0(it);
    const bool in_r1 = it < n1;
    const int lim_lo = in_r1 ? 0 : r2_lo;       // the staged range this tile belongs to
    const int lim_hi = in_r1 ? r1_hi : r2_hi;
    // does this tile hold any key visible to this wave's rows?
    const int t_lo = max(c0, lim_lo), t_hi = min(c0 + C::BN, lim_hi);
    const bool need = wave_live && ((t_lo < w1_hi) | ((t_lo < w2_hi) & (w2_lo < t_hi)));
    if (need) {
      if (in_r1 && c0 + C::BN - 1 < w_full) {
        tile_step<D, false>(Ks, Vt, qf, o, m, l, p.scale_log2, 0, 0, 0, 0, 0, j, hf);
      } else {
        // the row's visible intervals, clipped to this tile's key range
        const int lo_a = lim_lo, hi_a = min(hi1, lim_hi);
        const int lo_b = max(lo2, lim_lo), hi_b = min(hi2, lim_hi);
        tile_step<D, true>(Ks, Vt, qf, o, m, l, p.scale_log2, c0 + 4 * hf, lo_a, hi_a, lo_b,
                           hi_b, j, hf);
      }
    }

    __builtin_amdgcn_sched_barrier(0);
    if (it + 1 < ntiles) store_tile((it + 1) & 1);
    __syncthreads();
  }

  const float lt = l + __shfl_xor(l, 32);
  if (a >= p.twoL) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  bf16_t* orow = (bf16_t*)p.o + (((size_t)b * p.twoL + a) * p.Hq + h) * D;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 pk = {pack_bf16x2(o[i][4 * g] * inv, o[i][4 * g + 1] * inv),
                  pack_bf16x2(o[i][4 * g + 2] * inv, o[i][4 * g + 3] * inv)};
      *(u32x2*)(orow + 32 * i + 8 * g + 4 * hf) = pk;
    }
  }
  if (p.lse && hf == 0) p.lse[((size_t)b * p.Hq + h) * p.twoL + a] = (m + log2f(lt)) * kLn2;
}

// Heads per workgroup: the largest divisor of the GQA group size that is <= 8.
inline int heads_per_wg(int group) {
  for (int d = 8; d > 1; --d)
    if (group % d == 0) return d;
  return 1;
}

template <int D>
int launch_bf16(TwoStreamArgs a, hipStream_t st) {
  using C = Cfg<D>;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)two_stream_bf16_kernel<D>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS_BYTES);
    (void)hipGetLastError();
    attr_set = true;
  }
  // d = 64: one head x 4 row tiles per workgroup, so that three 4-wave
  // workgroups share a CU (the kernel is bound by vector-ALU softmax work and
  // needs the extra waves to hide latency). d = 128: the GQA heads sharing a
  // K/V head side by side (K/V staging is the larger cost there).
  a.gh = D == 64 ? 1 : heads_per_wg(a.group);
  a.nhc = a.group / a.gh;
  a.rt = D == 64 ? 4 : 8 / a.gh;
  a.nw = a.gh * a.rt;
  a.nqt = (a.twoL + 32 * a.rt - 1) / (32 * a.rt);
  const double nblocks = (double)a.batch * a.Hkv * a.nhc * a.nqt;
  if (nblocks >= 2147483647.0) return MARS_ERR_SHAPE;
  hipLaunchKernelGGL(two_stream_bf16_kernel<D>, dim3((unsigned)nblocks), dim3(64 * a.nw),
                     C::LDS_BYTES, st, a);
  return mars_launch_status();
}

template <int D>
int launch_f32(const TwoStreamArgs& a, hipStream_t st) {
  dim3 grid((a.twoL + 63) / 64, a.Hq, a.batch);
  hipLaunchKernelGGL(two_stream_f32_kernel<D>, grid, dim3(64), 0, st, a);
  return mars_launch_status();
}

}  // namespace

extern "C" int mars_attn_two_stream(const void* q, const void* k, const void* v, void* o,
                                    float* lse, int32_t batch, int32_t L, int32_t B,
                                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                    int32_t dtype, float softmax_scale, int32_t mask_mode,
                                    void* stream) {
  MARS_REQUIRE(q && k && v && o, MARS_ERR_NULL);
  MARS_REQUIRE(dtype == MARS_F32 || dtype == MARS_BF16, MARS_ERR_DTYPE);
  MARS_REQUIRE(batch >= 1 && L >= 1 && B >= 1 && B <= L && L <= (1 << 29), MARS_ERR_SHAPE);
  MARS_REQUIRE(n_q_heads >= 1 && n_kv_heads >= 1 && n_q_heads % n_kv_heads == 0, MARS_ERR_SHAPE);
  MARS_REQUIRE(mask_mode == 0 || mask_mode == 1, MARS_ERR_SHAPE);
  MARS_REQUIRE(head_dim >= 1, MARS_ERR_SHAPE);
  MARS_REQUIRE(mars_aligned16(q) && mars_aligned16(k) && mars_aligned16(v) &&
                   mars_aligned16(o) && mars_aligned16(lse),
               MARS_ERR_ALIGN);
  const int twoL = 2 * L;
  // Element offsets must fit the kernels' index arithmetic.
  MARS_REQUIRE((double)batch * twoL * n_q_heads * head_dim < 9.0e18, MARS_ERR_SHAPE);
  // Buffer loads address one (batch, head) slice with 32-bit byte offsets.
  MARS_REQUIRE(((double)twoL + 64) * n_q_heads * head_dim * 4 < 2147483647.0, MARS_ERR_SHAPE);

  TwoStreamArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.batch = batch;
  a.L = L;
  a.B = B;
  a.Hq = n_q_heads;
  a.Hkv = n_kv_heads;
  a.twoL = twoL;
  a.group = n_q_heads / n_kv_heads;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)head_dim);
  a.scale_log2 = scale * kLog2e;
  a.mask_mode = mask_mode;
  hipStream_t st = (hipStream_t)stream;

  if (dtype == MARS_BF16) {
    if (head_dim == 64) return launch_bf16<64>(a, st);
    if (head_dim == 128) return launch_bf16<128>(a, st);
    return MARS_ERR_UNSUPPORTED;
  }
  a.nqt = (twoL + 63) / 64;
  MARS_REQUIRE(n_q_heads <= 65535 && batch <= 65535, MARS_ERR_SHAPE);
  if (head_dim == 32) return launch_f32<32>(a, st);
  if (head_dim == 64) return launch_f32<64>(a, st);
  if (head_dim == 128) return launch_f32<128>(a, st);
  return MARS_ERR_UNSUPPORTED;
}
