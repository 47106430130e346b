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
#include <type_traits>

#include "attn_common.hpp"

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

__device__ __forceinline__ bool in_rows(int c, int hi1, int lo2, int hi2) {
  return (c < hi1) | ((c >= lo2) & (c < hi2));
}

// ---------------------------------------------------------------------------
// float32 path: one wave per 64 query rows, K/V staged in LDS 32 keys at a
// time, one query row per lane with its q and o rows in registers (at
// head_dim 128, 256 VGPRs + 135 accumulation registers: one wave per SIMD).
// A full-precision check path for the small fp32 configuration, not a fast one.
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
// Each wave owns 32 query rows of one query head. Scores are computed
// transposed, S^T = K Q^T, with the 32x32x16 MFMA: lane (j = l % 32,
// hf = l / 32) then holds query row j and 16 of the keys of each 32-key
// sub-tile, so a row reduction needs one exchange between the wave halves
// (v_permlane32_swap). The probabilities stay in registers and feed
// O^T = V^T P^T as the B operand: K slot (hf, e) of a 16-key chunk is key
// 4*hf + e (e < 4) or 8 + 4*hf + e - 4 (e >= 4), exactly the keys the lane
// holds. K and V tiles are plain row-major copies in LDS; the V^T fragments
// of the A operand come from the transposing LDS read ds_read_b64_tr_b16,
// which hands each lane one column (head dimension) of a 4-key x 16-column
// block that 16 lanes read as rows.
// ---------------------------------------------------------------------------
template <int D>
struct Cfg {
  static constexpr int BN = 64;            // keys per tile
  static constexpr int CPR = D / 8;        // 16-byte chunks per K or V row
  static constexpr int TSZ = BN * D;       // one K (or V) tile, elements
  static constexpr int NBLK = TSZ / 512;   // 1 KiB blocks per tile (one wave load each)
  static constexpr int BMAX = (NBLK + 3) / 4;  // blocks per wave, at >= 4 waves
};

// Rescaling of the running output is deferred until a row maximum grows by
// more than 2^8: until then exp2(s - m) stays below 256, which neither fp32
// nor bf16 minds, and the final O / l is unchanged by which m was used.
constexpr float kLazyRescale = 8.0f;

// One 64-key tile for one wave (32 query rows): S^T = K Q^T, online softmax,
// O^T += V^T P^T. Lane (j, hf) holds keys kb + 32n + 8(r/4) + (r%4) of its
// row. kad[c] / vad[i] are the lane's K and V^T read offsets inside a tile.
// masked (wave-uniform): only the keys whose bit is set in vm0 (half 0) or
// vm1 (half 1) count (bit 8 (r / 4) + r % 4 of a half is the lane's score r).
// Full and partial tiles share this one body, with the per-key test under a
// branch: as two inlined bodies, the two paths kept the output tuple in
// different registers, and every full tile copied all of it out and back
// (64 v_mov_b64 behind a wait for the last products) where they merged.
//
// The tile is worked as two 32-key halves in a software pipeline, so that a
// wave always has matrix work next to its vector work: the scores of half 1
// are multiplied while the probabilities of half 0 are formed, and half 0's
// P V products run while half 1's probabilities are formed. Each half keeps
// the lazy running maximum; when half 1 raises it, the output is rescaled
// after half 0's products (which were formed with the old maximum).
template <int D>
__device__ __forceinline__ void tile_step(const bf16_t* __restrict__ Ks,
                                          const bf16_t* __restrict__ Vs,
                                          const bf16x8 (&qf)[D / 16], f32x16 (&o)[D / 32],
                                          float& m, float& l, float cs, bool masked,
                                          uint32_t vm0, uint32_t vm1, const int (&kad)[D / 16],
                                          const int (&vad)[D / 32]) {
  auto qk = [&](int n) {
    f32x16 acc = f32x16{};
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const bf16x8 ka = *(const bf16x8*)(Ks + kad[c] + 32 * n * D);
      acc = mfma32(ka, qf[c], acc);
    }
    return acc;
  };
  auto mask = [&](f32x16& sv, int n) {
    if (masked) {
      // tie the mask to the scores so that the per-key tests are computed
      // after the products, not hoisted above them with every result held live
      uint32_t vm = n == 0 ? vm0 : vm1;
      asm volatile("" : "+v"(vm) : "v"(sv));
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[r] = (vm >> (8 * (r >> 2) + (r & 3))) & 1u ? sv[r] : -INFINITY;
    }
  };
  // row max of the raw scores, in log2 units (the scale is positive, so it
  // commutes with max)
  auto row_max = [&](const f32x16& sv) {
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sv[r]);
    return halves_max(mt) * cs;
  };
  // probabilities of 32 keys relative to the max -nm, as bf16 B fragments;
  // returns their fp32 sum
  auto probs = [&](const f32x16& sv, float nm, bf16x8& pa, bf16x8& pbk) {
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(fmaf(sv[r], cs, nm));
      ls += e;
      if (r < 8)
        pa[r] = (bf16_t)e;
      else
        pbk[r - 8] = (bf16_t)e;
    }
    return ls;
  };
  auto pv = [&](int kc, const bf16x8& pk) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      const bf16x4 vlo = lds_read_tr(Vs + vad[i] + 16 * kc * D);
      const bf16x4 vhi = lds_read_tr(Vs + vad[i] + (16 * kc + 8) * D);
      const bf16x8 va = {vlo[0], vlo[1], vlo[2], vlo[3], vhi[0], vhi[1], vhi[2], vhi[3]};
      o[i] = mfma32(va, pk, o[i]);
    }
  };

  // ---- half 0: scores, max; a growth rescales the earlier tiles' output
  f32x16 s0 = qk(0);
  mask(s0, 0);
  {
    const float mt = row_max(s0);
    const bool grow = mt > m + kLazyRescale;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float mnew = grow ? mt : m;
      // 1 when unchanged (also when still -inf), 0 when the first key arrives
      const float alpha = m == mnew ? 1.f : fast_exp2(m - mnew);
      l *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) o[i] *= alpha;
      m = mnew;
    }
  }
  // ---- half 1 scores | half 0 probabilities
  f32x16 s1 = qk(1);
  bf16x8 p0, p1;
  l += probs(s0, m == -INFINITY ? 0.f : -m, p0, p1);
  mask(s1, 1);
  const float mt1 = row_max(s1);
  const bool grow1 = mt1 > m + kLazyRescale;
  const bool any1 = __builtin_amdgcn_ballot_w64(grow1) != 0;
  const float m1 = grow1 ? mt1 : m;
  // ---- half 0 P V (old max) | half 1 probabilities (new max)
  pv(0, p0);
  pv(1, p1);
  bf16x8 p2, p3;
  const float l1 = probs(s1, m1 == -INFINITY ? 0.f : -m1, p2, p3);
  if (any1) {
    const float alpha = m == m1 ? 1.f : fast_exp2(m - m1);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) o[i] *= alpha;
    m = m1;
  }
  l += l1;
  // ---- half 1 P V
  pv(2, p2);
  pv(3, p3);
}

// Workgroup = nw waves, each owning one (query head, 32-row tile): gh heads of
// one GQA group x rt row tiles, so every K/V tile staged through LDS feeds
// 32 * nw query rows. The launcher uses gh = 1, rt = 4 at both head sizes.
// MODE is the mask: 0 the MARS two-stream mask, 1 plain causal over all 2L
// positions (a separate instance, so that the two modes are told apart in
// kernel traces and each folds its own interval arithmetic).
template <int D, int MODE>
__global__ __launch_bounds__(512, 2) void two_stream_bf16_kernel(TwoStreamArgs p) {
  using C = Cfg<D>;
  // two K/V stages (K tile then V tile), separate objects so that reads of
  // one stage are not ordered behind the direct loads filling the other
  __shared__ __attribute__((aligned(16))) bf16_t stage0[2 * C::TSZ];
  __shared__ __attribute__((aligned(16))) bf16_t stage1[2 * C::TSZ];
  const int NT = 64 * p.nw;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // d = 128 keeps the wave index in a scalar register (fewer vector registers
  // under its higher pressure); d = 64 measured faster with it in a VGPR
  const int w = D == 128 ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
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
  if (MODE == 0 && (p.L % bm) == 0) {
    const int nqs = p.L / bm;  // tiles per stream; clean tile i and mask tile i cost alike
    qt = (rank & 1) * nqs + (nqs - 1 - (rank >> 1));
  } else {
    qt = p.nqt - 1 - rank;
  }
  const int a0 = qt * bm;
  const int a_last = min(a0 + bm, p.twoL) - 1;

  // key ranges of the whole workgroup (what gets staged) and of this wave
  int r1_hi, r2_lo, r2_hi, full_below;
  rows_key_ranges(a0, a_last, p.L, p.B, MODE, r1_hi, r2_lo, r2_hi, full_below);
  const int n1 = (r1_hi + C::BN - 1) / C::BN;
  const int n2 = r2_hi > r2_lo ? (r2_hi - r2_lo + C::BN - 1) / C::BN : 0;
  const int ntiles = n1 + n2;
  const int wa0 = a0 + 32 * (w / p.gh);
  const bool wave_live = wa0 < p.twoL;
  const int wa_last = wave_live ? min(wa0 + 31, p.twoL - 1) : wa0;
  int w1_hi, w2_lo, w2_hi, w_full;
  rows_key_ranges(wa0, wa_last, p.L, p.B, MODE, w1_hi, w2_lo, w2_hi, w_full);

  // ---- this lane's query row and its visible key intervals ---------------
  const int a = wa0 + j;
  int hi1, lo2, hi2;
  row_intervals(a, p.L, p.B, MODE, hi1, lo2, hi2);

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

  auto tile_c0 = [&](int it) { return it < n1 ? it * C::BN : r2_lo + (it - n1) * C::BN; };

  // Direct global -> LDS loads: wave w fills 1 KiB blocks w, w + nw, ... of
  // the K and V tiles; lane l writes 16 bytes at block offset 16 l, which is
  // chunk slot l % CPR of row (block * 64 + l) / CPR, holding the global chunk
  // slot ^ swz(row). Rows past the end of the sequence read as zeros.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  auto issue_tile = [&](int it, bf16_t* st) {
    const int c0 = tile_c0(it);
#pragma unroll
    for (int i = 0; i < C::BMAX; ++i) {
      const int blk = wu + p.nw * i;
      if (blk < C::NBLK) {
        const int u = blk * 64 + lane;
        const int row = u / C::CPR, slot = u % C::CPR;
        const uint32_t rowb = (uint32_t)(((c0 + row) * rs) * sizeof(bf16_t));
        lds_load16(rk, st + blk * 512, rowb + 16 * (slot ^ swz_k<D>(row)));
        lds_load16(rv, st + C::TSZ + blk * 512, rowb + 16 * (slot ^ swz_v<D>(row)));
      }
    }
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  float m = -INFINITY, l = 0.f;

  // lane read offsets inside a tile. K: row j (+ 32 n), chunk 2c + hf.
  // V (transposing read): 16-lane group g = lane / 16 reads keys
  // 4 (g / 2) + lane % 16 / 4 (+ 16 kc, + 8) at head-dimension columns
  // 32 i + 16 (g % 2) + 4 (lane % 4), i.e. chunk 4 i + 2 (g % 2) + lane % 4 / 2.
  int kad[D / 16], vad[D / 32];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) kad[c] = j * D + 8 * ((2 * c + hf) ^ swz_k<D>(j));
  {
    const int vrow = 4 * hf + ((lane & 15) >> 2);
    const int vlow = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
      vad[i] = vrow * D + 8 * ((4 * i + vlow) ^ swz_v<D>(vrow)) + 4 * (lane & 1);
  }

  if (ntiles > 0) issue_tile(0, stage0);
  // The query fragments must have landed before the loop: otherwise the
  // wait-count bookkeeping treats them as in flight on every iteration and
  // each tile would stall on its own prefetch.
#pragma unroll
  for (int c = 0; c < D / 16; ++c) asm volatile("" ::"v"(qf[c]));
  __syncthreads();

  // one tile; the LDS stage is a compile-time constant so that every LDS
  // address is a lane offset plus an immediate
  auto iteration = [&](int it, auto stage_tag) {
    constexpr int STG = decltype(stage_tag)::value;
    if (it + 1 < ntiles) issue_tile(it + 1, STG == 0 ? stage1 : stage0);
    // keep the prefetch issued before the compute
    __builtin_amdgcn_sched_barrier(0);

    const bf16_t* Ks = STG == 0 ? stage0 : stage1;
    const bf16_t* Vs = Ks + C::TSZ;
    const int c0 = tile_c0(it);
    const bool in_r1 = it < n1;
    const int lim_lo = in_r1 ? 0 : r2_lo;       // the staged range this tile belongs to
    const int lim_hi = in_r1 ? r1_hi : r2_hi;
    // does this tile hold any key visible to this wave's rows?
    const int t_lo = max(c0, lim_lo), t_hi = min(c0 + C::BN, lim_hi);
    const bool need = wave_live && ((t_lo < w1_hi) | ((t_lo < w2_hi) & (w2_lo < t_hi)));
    if (need) {
      const bool full = in_r1 && c0 + C::BN - 1 < w_full;  // wave-uniform
      uint32_t vm0 = 0u, vm1 = 0u;
      if (!full) {
        // the row's visible intervals clipped to the staged range, as one bit
        // mask per 32-key half (bit t: key t of the half past the lane's first
        // key kb). One masked code path serves every partial tile: per-kind
        // copies (upper bound, range, both) held 43 more VGPRs at d = 64.
        const int kb = c0 + 4 * hf;
        const int hi_a = min(hi1, lim_hi) - kb;
        const int lo_b = max(lo2, lim_lo) - kb;
        const int hi_b = min(hi2, lim_hi) - kb;
        vm0 = row_bits(0, hi_a) | row_bits(lo_b, hi_b);
        vm1 = row_bits(-32, hi_a - 32) | row_bits(lo_b - 32, hi_b - 32);
      }
      tile_step<D>(Ks, Vs, qf, o, m, l, p.scale_log2, !full, vm0, vm1, kad, vad);
    }

    // the next stage has landed (the barrier waits for this wave's direct
    // loads) and every wave is done reading this one
    __syncthreads();
  };
  for (int it = 0; it < ntiles; it += 2) {
    iteration(it, std::integral_constant<int, 0>{});
    if (it + 1 < ntiles) iteration(it + 1, std::integral_constant<int, 1>{});
  }

  const float lt = halves_sum(l);
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

template <int D>
int launch_bf16(TwoStreamArgs a, hipStream_t st) {
  using C = Cfg<D>;
  // One head x 4 row tiles per workgroup at both head sizes: four 4-wave
  // workgroups share a CU at d = 64 (123 VGPRs, 32 KiB of LDS each), two at
  // d = 128 (200 VGPRs; the kernel is bound by latency and needs the waves
  // resident). At d = 128 this measured 8% faster
  // than packing the 7 GQA heads of a K/V head into one 7-wave workgroup,
  // which left one SIMD of every CU with a single wave; the heads of a K/V head
  // still run side by side on one XCD and share its L2.
  a.gh = 1;
  a.nhc = a.group / a.gh;
  a.rt = 4;
  a.nw = a.gh * a.rt;
  a.nqt = (a.twoL + 32 * a.rt - 1) / (32 * a.rt);
  const double nblocks = (double)a.batch * a.Hkv * a.nhc * a.nqt;
  if (nblocks >= 2147483647.0) return MARS_ERR_SHAPE;
  if (a.mask_mode == 0)
    hipLaunchKernelGGL((two_stream_bf16_kernel<D, 0>), dim3((unsigned)nblocks),
                       dim3(64 * a.nw), 0, st, a);
  else
    hipLaunchKernelGGL((two_stream_bf16_kernel<D, 1>), dim3((unsigned)nblocks),
                       dim3(64 * a.nw), 0, st, a);
  return mars_launch_status();
}

template <int D>
int launch_f32(const TwoStreamArgs& a, hipStream_t st) {
  dim3 grid((a.twoL + 63) / 64, a.Hq, a.batch);
  hipLaunchKernelGGL(two_stream_f32_kernel<D>, grid, dim3(64), 0, st, a);
  return mars_launch_status();
}

}  // namespace

namespace {
// Common path of both entry points: the attention over n = twoL positions under
// mask_mode (0: MARS two-stream mask with stream length L and block size B,
// 1: causal over all n positions).
int run_attention(const void* q, const void* k, const void* v, void* o, float* lse, int32_t batch,
                  int32_t L, int32_t twoL, int32_t B, int32_t n_q_heads, int32_t n_kv_heads,
                  int32_t head_dim, int32_t dtype, float softmax_scale, int32_t mask_mode,
                  void* stream) {
  MARS_REQUIRE(q && k && v && o, MARS_ERR_NULL);
  MARS_REQUIRE(dtype == MARS_F32 || dtype == MARS_BF16, MARS_ERR_DTYPE);
  MARS_REQUIRE(n_q_heads >= 1 && n_kv_heads >= 1 && n_q_heads % n_kv_heads == 0, MARS_ERR_SHAPE);
  MARS_REQUIRE(head_dim >= 1, MARS_ERR_SHAPE);
  MARS_REQUIRE(mars_aligned16(q) && mars_aligned16(k) && mars_aligned16(v) &&
                   mars_aligned16(o) && mars_aligned16(lse),
               MARS_ERR_ALIGN);
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
}  // namespace

extern "C" int mars_attn_two_stream(const void* q, const void* k, const void* v, void* o,
                                    float* lse, int32_t batch, int32_t L, int32_t B,
                                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                    int32_t dtype, float softmax_scale, int32_t mask_mode,
                                    void* stream) {
  MARS_REQUIRE(q && k && v && o, MARS_ERR_NULL);
  MARS_REQUIRE(dtype == MARS_F32 || dtype == MARS_BF16, MARS_ERR_DTYPE);
  MARS_REQUIRE(batch >= 1 && L >= 1 && B >= 1 && B <= L && L <= (1 << 29), MARS_ERR_SHAPE);
  MARS_REQUIRE(mask_mode == 0 || mask_mode == 1, MARS_ERR_SHAPE);
  return run_attention(q, k, v, o, lse, batch, L, 2 * L, B, n_q_heads, n_kv_heads, head_dim,
                       dtype, softmax_scale, mask_mode, stream);
}

extern "C" int mars_attn_causal(const void* q, const void* k, const void* v, void* o, float* lse,
                                int32_t batch, int32_t T, int32_t n_q_heads, int32_t n_kv_heads,
                                int32_t head_dim, int32_t dtype, float softmax_scale,
                                void* stream) {
  MARS_REQUIRE(q && k && v && o, MARS_ERR_NULL);
  MARS_REQUIRE(dtype == MARS_F32 || dtype == MARS_BF16, MARS_ERR_DTYPE);
  MARS_REQUIRE(batch >= 1 && T >= 1 && T <= (1 << 30), MARS_ERR_SHAPE);
  // causal mode: the stream split (L, B) plays no part
  return run_attention(q, k, v, o, lse, batch, (T + 1) / 2, T, 1, n_q_heads, n_kv_heads,
                       head_dim, dtype, softmax_scale, 1, stream);
}
