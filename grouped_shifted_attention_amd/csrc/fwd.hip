// S2-Attn forward kernels for gfx950.
//
// One workgroup computes BM rows (a "q tile") of one unit (batch b, q head h,
// group g); each wave owns 32 rows of the tile.  The unit's local row j
// lives at original position (g*G + j + shift_h) mod N, so the roll by
// -shift_h and the cut into groups are only address arithmetic (AIMech
// "LongLoRA and Shifted Sparse Attention (S^2-Attn)", opening definition);
// the output row is written back to the same original position, which is
// the roll back by +shift_h.
//
// Per k/v tile of BN = 64 keys, staged in LDS (double-buffered):
//   S^T = K Q^T           MFMA, A = K rows from LDS, B = Q held in VGPRs
//   causal mask           only on tiles that cross the wave's diagonal
//   online softmax        exp2 domain; row max/sum need one lane swap (l^32)
//   O^T += V^T P^T        MFMA, A = V^T read transposed (ds_read_b64_tr_b16)
//                         from the row-major V tile, B = P taken straight
//                         from the S^T accumulators
// Computing S^T (not S) leaves each lane with one query row, so the softmax
// statistics and the rescale of O are per-lane scalars.
//
// Groups of up to 2048 rows: fwd_kernel, 2 or 4 waves, tiles loaded straight
// into LDS.  Longer groups: fwd_pp_kernel, 8 waves in two groups whose
// matrix and softmax phases alternate on each SIMD.
#include "device_common.hpp"
#include "kernels.hpp"
#include "staging.hpp"

#include <type_traits>

namespace s2a {

namespace {

constexpr int kBN = 64;
constexpr float kLazy = 8.f;  // log2-domain slack before the softmax reference moves

// RB row blocks of 32 query rows per wave (the launcher uses RB = 1, two
// waves per SIMD; RB = 2 would let each K/V fragment feed two MFMAs but
// needs more registers than one wave per SIMD leaves without spilling).
template <int D, int NW, int RB, bool ROPE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(RB == 2 ? 1 : 2, RB == 2 ? 1 : 2))) void fwd_kernel(FwdArgs a, RopeTable rope) {
  constexpr int BM = NW * 32 * RB;
  using TileStage = LdsStage<D, kBN, NW>;
  // Double-buffered K/V tiles (tile n in buffer n & 1), each buffer two
  // distinct LDS objects named at compile time: the compiler can then tell
  // the reads of one buffer from the loads filling the other and does not
  // make the reads wait for a tile still in flight.
  __shared__ __attribute__((aligned(16))) uint16_t Ks0[TileStage::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Ks1[TileStage::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs0[TileStage::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs1[TileStage::ELEMS];
  auto kbuf = [&](auto c) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(c)::value) return Ks1; else return Ks0;
  };
  auto vbuf = [&](auto c) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(c)::value) return Vs1; else return Vs0;
  };
  using P0 = std::false_type;
  using P1 = std::true_type;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it scalar
  const int lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const TileLane<D> sw(lane);
  const Shape& s = a.s;

  // Work item: heavy (long causal rows) tiles first within a unit; units
  // contiguous per XCD.
  const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const int unit = logical / a.tiles;
  const int t = a.tiles - 1 - (logical - unit * a.tiles);
  const QUnit uq = decode_q_unit(unit, s);
  const int g = uq.g, h = uq.h, b = uq.b;
  const int sh = head_shift(h, s);
  const int kvh = h / (s.H / s.Hkv);
  const int base = g * s.G + sh;
  const long long kv_row = (long long)s.Hkv * D;
  const uint16_t* kb_ptr = a.k + (long long)b * s.N * kv_row + (long long)kvh * D;
  const uint16_t* vb_ptr = a.v + (long long)b * s.N * kv_row + (long long)kvh * D;

  // ---- this lane's query rows (one per row block), held as MFMA B operands ----
  const int wave_q0 = t * BM + wave * 32 * RB;
  int qi[RB], qpos[RB];
  bool qvalid[RB];
  long long qoff[RB];
  // The softmax scale and log2(e) are folded into q once (one bf16
  // rounding of q * scale * log2 e), so S^T comes out of the MFMA in log2
  // units and P = exp2(S - m) needs no multiply.
  bf16x8 qf[RB][D / 16];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    qi[rb] = wave_q0 + rb * 32 + l32;
    qvalid[rb] = qi[rb] < s.G;
    qpos[rb] = qvalid[rb] ? orig_pos(base, qi[rb], s.N) : 0;
    qoff[rb] = ((long long)(b * (long long)s.N + qpos[rb]) * s.H + h) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const u32x4 raw = qvalid[rb] ? ld16(a.q + qoff[rb] + kk * 16 + hh * 8) : zero_u4();
      float x[8];
      unpack8(raw, x);
      if constexpr (ROPE) rope_rotate8(x, qpos[rb], rope.rev, kk * 16 + hh * 8, false);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= a.scale_log2;
      qf[rb][kk] = as_bf16x8(pack8(x));
    }
  }

  f32x16 o[RB][D / 32];
  // Softmax reference m_run (log2 units, -inf before the first tile).  The
  // S^T accumulators start at s0 = -m_run (0 before the first tile), so the
  // MFMA hands back S - m_run and P = exp2 of it.
  float m_run[RB], l_run[RB];  // l_run: this lane's half of the running row sum
  f32x16 s0[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) o[rb][i] = zero16();
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
    s0[rb] = zero16();
  }

  const int rows_end = min((t + 1) * BM, s.G);
  const int ntiles = (rows_end + kBN - 1) / kBN;

  const TileStage ts(wave, lane, (int)kv_row);
  // K and V tiles go straight from global memory into the padded LDS tiles;
  // rows past the group end point at the group's last row (their keys are
  // masked, so the values never contribute).
  auto load_tile = [&](int n, auto c) __attribute__((always_inline)) {
    const int key0 = n * kBN;
    const uint16_t* kt = contig_tile(kb_ptr, kv_row, base, key0, kBN, s.G, s.N);
    if (kt != nullptr) {
      ts.load_contig(kt, kbuf(c), wave);
      ts.load_contig(vb_ptr + (kt - kb_ptr), vbuf(c), wave);
    } else {
      auto rows = [&](const uint16_t* head0) {
        return [=, &s](int row) {
          const int j = min(key0 + row, s.G - 1);
          return head0 + orig_pos(base, j, s.N) * kv_row;
        };
      };
      ts.load_rows(rows(kb_ptr), kbuf(c), wave, lane);
      ts.load_rows(rows(vb_ptr), vbuf(c), wave, lane);
    }
  };

  // Tiles whose keys all precede this wave's first row need no mask; the
  // rest (the diagonal, and for the lower row blocks one tile wholly above
  // them, which the mask zeroes) do.
  const int n_full = min(ntiles, (wave_q0 + 1) / kBN);

  // One k/v tile: S^T = K Q^T, online softmax, O^T += V^T P^T for each row
  // block.  MASK only for the tiles from n_full on.
  auto compute = [&](int n, auto mask_tag, auto c) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int NB = kBN / 32;  // 32-key blocks per tile
    const int key0 = n * kBN;
    // S^T: each K fragment (one per 32-key block and k-step) is read once
    // and feeds one MFMA per row block; the 2*RB accumulators are
    // independent, so back-to-back MFMAs never wait on each other.
    f32x16 sc[RB][NB];
    {
      const uint16_t* kt = kbuf(c);
      constexpr int KD = 3;  // K fragments in flight: reads run two k-steps ahead
      bf16x8 kf[KD][NB];
#pragma unroll
      for (int kk = 0; kk < KD - 1; ++kk)
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) kf[kk][kb] = sw.row(kt, kb * 32, kk);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        if (kk + KD - 1 < D / 16) {
#pragma unroll
          for (int kb = 0; kb < NB; ++kb) kf[(kk + KD - 1) % KD][kb] = sw.row(kt, kb * 32, kk + KD - 1);
        }
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            sc[rb][kb] = mfma32x32x16(kf[kk % KD][kb], qf[rb][kk], kk == 0 ? s0[rb] : sc[rb][kb]);
      }
      // Keep the K reads (KD-1) k-steps ahead of the MFMAs that use them:
      // the scheduler would otherwise sink each read next to its use and
      // expose the LDS latency.
      __builtin_amdgcn_sched_group_barrier(0x100, (KD - 1) * NB, 0);
#pragma unroll
      for (int i = 0; i < (D / 16) * NB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, RB, 0);
        if (i < (D / 16 - (KD - 1)) * NB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    bf16x8 pb[RB][NB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if constexpr (MASK) {
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = key0 + kb * 32 + acc_row(r, hh);
            if (j > qi[rb]) sc[rb][kb][r] = -INFINITY;
          }
      }
      // Online softmax in the exp2 domain with a lazily moved reference: the
      // reference moves (and O, l are rescaled) only when some row's max
      // exceeds it by more than kLazy (so p <= 2^kLazy), and on the first
      // tile; otherwise the stale reference stays, which changes nothing in
      // exact arithmetic.
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[rb][kb][r]);
      mx = half_max(mx);  // relative to m_run (absolute before the first tile)
      const bool first = m_run[rb] == -INFINITY;
      if (__any(mx > kLazy || first)) {
        float m_new = first ? mx : m_run[rb] + fmaxf(mx, 0.f);
        if (mx == -INFINITY) m_new = m_run[rb];  // nothing visible yet
        const float alpha = m_new == m_run[rb] ? 1.f : fast_exp2(m_run[rb] - m_new);
        const float shift = m_new == -INFINITY ? 0.f : m_new - (first ? 0.f : m_run[rb]);
        m_run[rb] = m_new;
        l_run[rb] *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) o[rb][i] *= alpha;
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[rb][kb][r] -= shift;
        const float neg = m_run[rb] == -INFINITY ? 0.f : -m_run[rb];
#pragma unroll
        for (int r = 0; r < 16; ++r) s0[rb][r] = neg;
      }
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = fast_exp2(sc[rb][kb][r]);
          sc[rb][kb][r] = pv;
          rs += pv;
        }
      l_run[rb] += rs;
      // P as bf16 B operands: accumulator elements 0..7 and 8..15 of each
      // 32-key block are the two 16-key halves of the reduction.
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        pb[rb][kb][0] = cvt8(f32x8{sc[rb][kb][0], sc[rb][kb][1], sc[rb][kb][2], sc[rb][kb][3],
                                   sc[rb][kb][4], sc[rb][kb][5], sc[rb][kb][6], sc[rb][kb][7]});
        pb[rb][kb][1] = cvt8(f32x8{sc[rb][kb][8], sc[rb][kb][9], sc[rb][kb][10], sc[rb][kb][11],
                                   sc[rb][kb][12], sc[rb][kb][13], sc[rb][kb][14], sc[rb][kb][15]});
      }
    }
    // O^T += V^T P^T: each V^T fragment (read through the transposing read
    // from the row-major V tile, one step ahead) feeds one MFMA per row
    // block; the D/32 * RB output blocks are independent accumulators.
    {
      const uint16_t* vt = vbuf(c);
      constexpr int KS = kBN / 16;  // 16-key reduction steps per tile
      bf16x8 vf[2][D / 32];
#pragma unroll
      for (int db = 0; db < D / 32; ++db) vf[0][db] = sw.tr(vt, 0, db);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) {
#pragma unroll
          for (int db = 0; db < D / 32; ++db) vf[(ks + 1) & 1][db] = sw.tr(vt, (ks + 1) * 16, db);
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            o[rb][db] = mfma32x32x16(vf[ks & 1][db], pb[rb][ks >> 1][ks & 1], o[rb][db]);
      }
    }
  };

  // Step n (buffer n & 1): start loading tile n+1 (into the other buffer,
  // or into VGPRs written to it at the end), compute tile n, wait for tile
  // n+1 and meet at the barrier.  Every wave runs ntiles steps, so the
  // barriers match.
  auto step = [&](int n, auto mask_tag, auto c) __attribute__((always_inline)) {
    using Next = std::integral_constant<bool, !decltype(c)::value>;
    if (n + 1 < ntiles) load_tile(n + 1, Next{});
    compute(n, mask_tag, c);
    wait_vmem_all();
    lds_barrier();
  };
  // Steps n .. n1-1, unrolled by two so each names its buffer statically.
  auto run = [&](int n, int n1, auto mask_tag) __attribute__((always_inline)) {
    if (n < n1 && (n & 1)) step(n++, mask_tag, P1{});
    for (; n + 1 < n1; n += 2) {
      step(n, mask_tag, P0{});
      step(n + 1, mask_tag, P1{});
    }
    if (n < n1) step(n, mask_tag, P0{});
  };

  load_tile(0, P0{});
  wait_vmem_all();
  lds_barrier();
  run(0, n_full, std::false_type{});
  run(n_full, ntiles, std::true_type{});

  // ---- epilogue: normalise, write O and LSE at the original position ----
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float lt = half_sum(l_run[rb]);
    const float inv = 1.f / lt;
    if (qvalid[rb]) {
      uint16_t* op = a.out + qoff[rb];
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d = db * 32 + r4 * 8 + hh * 4;
          st8(op + d, cvt4_bits(o[rb][db][r4 * 4] * inv, o[rb][db][r4 * 4 + 1] * inv,
                                o[rb][db][r4 * 4 + 2] * inv, o[rb][db][r4 * 4 + 3] * inv));
        }
      if (hh == 0 && a.lse != nullptr)
        a.lse[((long long)b * s.H + h) * s.N + qpos[rb]] = (m_run[rb] + __log2f(lt)) * kLn2;
    }
  }
}

// Long groups: eight waves of 32 query rows (BM = 256) in two groups of
// four, X = waves 0-3 and Y = waves 4-7, one wave of each per SIMD.  A wave's
// work per k/v tile m splits into a matrix phase (O^T += V(m-1)^T P(m-1)^T,
// then S^T(m) = K(m) Q^T) and a softmax phase (mask, statistics,
// P(m) = exp2(S^T(m)), bf16 pack).  The groups run these phases one slot
// apart, slots being separated by workgroup barriers:
//   slot 2m:    X: matrix phase m          Y: softmax phase m-1
//   slot 2m+1:  X: softmax phase m         Y: matrix phase m
// so each SIMD's matrix core works while its other wave is busy on the
// vector ALU, instead of both waves waiting on the same unit at once.
// X stages the K tiles and Y the V tiles through VGPRs: tile m+1 is loaded
// at the start of the wave's matrix phase m and written to LDS at the start
// of its softmax phase m (the writes then drain under the VALU work).  Tile n
// sits in buffer n & 1.  K(m+1) (written in slot 2m+1) replaces K(m-1), last
// read in slot 2m-1; V(m+1) (slot 2m+2) replaces V(m-1), last read in slot
// 2m+1; each is first read two slots after its write, past the barrier that
// ends the write slot.
template <int D, bool ROPE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_pp_kernel(FwdArgs a, RopeTable rope) {
  constexpr int BM = 256;
  constexpr int RS = D + 8;
  constexpr int TE = kBN * RS;  // elements of one padded tile
  constexpr int NB = kBN / 32;  // 32-key blocks per tile
  __shared__ __attribute__((aligned(16))) uint16_t Ks0[TE];
  __shared__ __attribute__((aligned(16))) uint16_t Ks1[TE];
  __shared__ __attribute__((aligned(16))) uint16_t Vs0[TE];
  __shared__ __attribute__((aligned(16))) uint16_t Vs1[TE];
  auto kbuf = [&](auto c) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(c)::value) return Ks1; else return Ks0;
  };
  auto vbuf = [&](auto c) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(c)::value) return Vs1; else return Vs0;
  };
  using P0 = std::false_type;
  using P1 = std::true_type;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: X, 1: Y
  const int lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const TileLane<D> sw(lane);
  const Shape& s = a.s;

  const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const int unit = logical / a.tiles;
  const int t = a.tiles - 1 - (logical - unit * a.tiles);
  const QUnit uq = decode_q_unit(unit, s);
  const int g = uq.g, h = uq.h, b = uq.b;
  const int sh = head_shift(h, s);
  const int kvh = h / (s.H / s.Hkv);
  const int base = g * s.G + sh;
  const long long kv_row = (long long)s.Hkv * D;
  const uint16_t* kb_ptr = a.k + (long long)b * s.N * kv_row + (long long)kvh * D;
  const uint16_t* vb_ptr = a.v + (long long)b * s.N * kv_row + (long long)kvh * D;

  // This lane's query row, held as MFMA B operands, prescaled by
  // scale * log2(e) (one bf16 rounding).
  const int wave_q0 = t * BM + wave * 32;
  const int qi = wave_q0 + l32;
  const bool qvalid = qi < s.G;
  const int qpos = qvalid ? orig_pos(base, qi, s.N) : 0;
  const long long qoff = ((long long)(b * (long long)s.N + qpos) * s.H + h) * D;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const u32x4 raw = qvalid ? ld16(a.q + qoff + kk * 16 + hh * 8) : zero_u4();
    float x[8];
    unpack8(raw, x);
    if constexpr (ROPE) rope_rotate8(x, qpos, rope.rev, kk * 16 + hh * 8, false);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] *= a.scale_log2;
    qf[kk] = as_bf16x8(pack8(x));
  }

  // O^T accumulators, softmax reference m_run (log2 units; -inf before the
  // first tile) and this lane's half of the row sum.  S^T accumulators start
  // at s0 = -m_run, so the MFMA returns S - m_run.
  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = zero16();
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 s0 = zero16();
  f32x16 sc[NB];
  bf16x8 pb[NB][2];

  const int rows_end = min((t + 1) * BM, s.G);
  const int T = (rows_end + kBN - 1) / kBN;
  // Tiles before n_full lie wholly left of this wave's diagonal.
  const int n_full = min(T, (wave_q0 + 1) / kBN);
  // Key-tile walk direction.  When a unit's workgroups fit on one XCD's CUs,
  // they either start together (the first unit on an XCD, and each unit after
  // one whose workgroups all ended together) or one after another as the
  // previous unit's shorter workgroups end, the longest first.  Walking up
  // from key 0 keeps the first kind on the same k/v tile at the same time,
  // walking down from the diagonal does so for the second (each then ends
  // together), so alternating the direction between consecutive units lets a
  // unit's workgroups share each k/v tile in L2 instead of re-reading the
  // head's k/v rows from HBM at staggered times.  Units of more workgroups
  // than an XCD has CUs keep walking up, which re-reads less for them.
  const bool walk_down = a.tiles <= kCusPerXcd && (unit & 1) != 0;
  auto tile_at = [&](int i) __attribute__((always_inline)) { return walk_down ? T - 1 - i : i; };

  // ---- matrix phase ----
  // S^T(m) = K(m) Q^T: K fragments read (KD - 1) k-steps ahead of their
  // MFMAs.  O^T += V^T P^T: the V^T fragments of the next 16-key step are read
  // while the current step's MFMAs run; the first step's fragments are read at
  // the end of the preceding softmax phase, where the wave would otherwise
  // idle at the barrier.  Scheduling groups pin the read / MFMA order (the
  // scheduler would otherwise sink each read next to its use).
  auto vfrag = [&](const uint16_t* vt, int f) __attribute__((always_inline)) {
    return sw.tr(vt, (f / (D / 32)) * 16, f % (D / 32));
  };
  auto mat_s = [&](const uint16_t* kt) __attribute__((always_inline)) {
    constexpr int KD = 3;  // K fragments in flight: reads run two k-steps ahead
    bf16x8 kf[KD][NB];
#pragma unroll
    for (int kk = 0; kk < KD - 1; ++kk)
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) kf[kk][kb] = sw.row(kt, kb * 32, kk);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      if (kk + KD - 1 < D / 16) {
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) kf[(kk + KD - 1) % KD][kb] = sw.row(kt, kb * 32, kk + KD - 1);
      }
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) sc[kb] = mfma32x32x16(kf[kk % KD][kb], qf[kk], kk == 0 ? s0 : sc[kb]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, (KD - 1) * NB, 0);
#pragma unroll
    for (int i = 0; i < (D / 16) * NB; ++i) {
      if (i < (D / 16 - (KD - 1)) * NB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  };
  bf16x8 vpre[D / 32];  // first V^T fragments of the next PV, read at the start of the softmax phase
  auto mat_pv = [&](const uint16_t* vt) __attribute__((always_inline)) {
    constexpr int KS = kBN / 16;
    bf16x8 vf[2][D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) vf[0][db] = vpre[db];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        if (ks + 1 < KS) vf[(ks + 1) & 1][db] = vfrag(vt, (ks + 1) * (D / 32) + db);
        o[db] = mfma32x32x16(vf[ks & 1][db], pb[ks >> 1][ks & 1], o[db]);
      }
    }
#pragma unroll
    for (int i = 0; i < KS * (D / 32); ++i) {
      if (i < (KS - 1) * (D / 32)) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  };

  // ---- softmax phase for tile n ----
  auto softmax = [&](int n) __attribute__((always_inline)) {
    if (n >= n_full) {
      const int key0 = n * kBN;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key0 + kb * 32 + acc_row(r, hh) > qi) sc[kb][r] = -INFINITY;
    }
    // The reference moves (and O, l are rescaled) only on the first tile or
    // when some row's max exceeds it by more than kLazy.
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
    mx = half_max(mx);
    const bool first = m_run == -INFINITY;
    if (__any(mx > kLazy || first)) {
      float m_new = first ? mx : m_run + fmaxf(mx, 0.f);
      if (mx == -INFINITY) m_new = m_run;
      const float alpha = m_new == m_run ? 1.f : fast_exp2(m_run - m_new);
      const float shift = m_new == -INFINITY ? 0.f : m_new - (first ? 0.f : m_run);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) o[i] *= alpha;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kb][r] -= shift;
      const float neg = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
      for (int r = 0; r < 16; ++r) s0[r] = neg;
    }
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = fast_exp2(sc[kb][r]);
        sc[kb][r] = pv;
        rs += pv;
      }
    l_run += rs;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      pb[kb][0] = cvt8(f32x8{sc[kb][0], sc[kb][1], sc[kb][2], sc[kb][3], sc[kb][4], sc[kb][5], sc[kb][6], sc[kb][7]});
      pb[kb][1] = cvt8(f32x8{sc[kb][8], sc[kb][9], sc[kb][10], sc[kb][11], sc[kb][12], sc[kb][13], sc[kb][14], sc[kb][15]});
    }
  };

  // ---- staging: X stages K tiles, Y stages V tiles, through VGPRs ----
  // Thread tg of a group owns 16-byte chunks tg, tg + 256, ... of the tile
  // (chunk = tile row * D/8 + column chunk).
  constexpr int kCh = D / 8;
  constexpr int kPer = kBN * kCh / 256;
  static_assert(kBN * kCh % 256 == 0, "whole chunks per thread");
  const int tg = tid & 255;
  const uint16_t* my_src = grp ? vb_ptr : kb_ptr;
  u32x4 stg[kPer];
  // Element offset of each owned chunk inside a tile of consecutive rows
  // (fits in 32 bits: the host rejects shapes with 64 * Hkv * D >= 2^31).
  int roff[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int item = tg + i * 256;
    roff[i] = (item / kCh) * (int)kv_row + (item % kCh) * 8;
  }
  // A tile of consecutive rows (all but the tiles that reach past the group
  // end or wrap round the sequence end) costs one address add per chunk.
  auto gload = [&](int n) __attribute__((always_inline)) {
    const int key0 = n * kBN;
    const uint16_t* tile = contig_tile(my_src, kv_row, base, key0, kBN, s.G, s.N);
    if (tile != nullptr) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) stg[i] = ld16(tile + roff[i]);
    } else {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int item = tg + i * 256;
        const int row = item / kCh, col = (item % kCh) * 8;
        stg[i] = ld16(my_src + orig_pos(base, min(key0 + row, s.G - 1), s.N) * kv_row + col);
      }
    }
  };
  auto swrite = [&](uint16_t* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int item = tg + i * 256;
      st16(dst + (item / kCh) * RS + (item % kCh) * 8, stg[i]);
    }
  };

  // Slot boundary: nothing is scheduled across it, so each phase keeps its
  // own instructions.
  auto slot_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // Every wave runs the same sequence -- matrix phase of tile m, barrier,
  // softmax phase of tile m, barrier -- and Y starts it one slot later than
  // X (one extra barrier up front).
  // Matrix phase m has no PV part for m = 0 and only the PV part for m = T.
  auto step = [&](int m, auto c) __attribute__((always_inline)) {
    using Cn = std::integral_constant<bool, !decltype(c)::value>;
    // Issued in every step (the last re-reads the final tile, still in L2),
    // so no branch sits around the loads and the wait before the staging
    // write counts only them.
    gload(tile_at(min(m + 1, T - 1)));
    if (m >= 1) mat_pv(vbuf(Cn{}));
    if (m < T) mat_s(kbuf(c));
    if (m < T) slot_barrier();
    if (m < T) {
      // The staged tile and the first V(m) fragments go to LDS first, so
      // they drain during the VALU work instead of holding up the barrier.
      // The target buffer held tile m-1, whose last reader (the other
      // group's matrix phase) ended at the previous slot boundary.
      if (m + 1 < T) swrite(grp ? vbuf(Cn{}) : kbuf(Cn{}));
#pragma unroll
      for (int db = 0; db < D / 32; ++db) vpre[db] = vfrag(vbuf(c), db);  // V(m): visible since its write slot ended
      softmax(tile_at(m));
      if (grp == 0 || m + 1 < T) slot_barrier();
    }
  };
  gload(tile_at(0));
  swrite(grp ? Vs0 : Ks0);
  slot_barrier();
  if (grp) slot_barrier();
  for (int m = 0; m <= T; m += 2) {
    step(m, P0{});
    if (m + 1 <= T) step(m + 1, P1{});
  }

  // ---- epilogue: normalise, write O and LSE at the original position ----
  const float lt = half_sum(l_run);
  const float inv = 1.f / lt;
  if (qvalid) {
    uint16_t* op = a.out + qoff;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = db * 32 + r4 * 8 + hh * 4;
        st8(op + d, cvt4_bits(o[db][r4 * 4] * inv, o[db][r4 * 4 + 1] * inv, o[db][r4 * 4 + 2] * inv,
                              o[db][r4 * 4 + 3] * inv));
      }
    if (hh == 0 && a.lse != nullptr) a.lse[((long long)b * s.H + h) * s.N + qpos] = (m_run + __log2f(lt)) * kLn2;
  }
}

template <int D, bool ROPE>
hipError_t launch_fwd_pp(FwdArgs a, const RopeTable* rope, hipStream_t stream) {
  a.tiles = (a.s.G + 255) / 256;
  const long long grid = (long long)a.s.B * a.s.H * a.s.NG * a.tiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  RopeTable rt{};
  if (ROPE) rt = *rope;
  hipLaunchKernelGGL((fwd_pp_kernel<D, ROPE>), dim3((unsigned)grid), dim3(512), 0, stream, a, rt);
  return hipGetLastError();
}

template <int D, int NW, int RB, bool ROPE>
hipError_t launch_fwd_t(FwdArgs a, const RopeTable* rope, hipStream_t stream) {
  constexpr int BM = NW * 32 * RB;
  a.tiles = (a.s.G + BM - 1) / BM;
  const long long grid = (long long)a.s.B * a.s.H * a.s.NG * a.tiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  RopeTable rt{};
  if (ROPE) rt = *rope;
  hipLaunchKernelGGL((fwd_kernel<D, NW, RB, ROPE>), dim3((unsigned)grid), dim3(NW * 64), 0, stream, a, rt);
  return hipGetLastError();
}

template <int D, bool ROPE>
hipError_t launch_fwd_d(const FwdArgs& a, const RopeTable* rope, hipStream_t stream) {
  if (a.s.G <= 64) return launch_fwd_t<D, 2, 1, ROPE>(a, rope, stream);
  // Up to 2048 rows the 4-wave kernel, with twice the workgroups, finishes
  // first (about 9% at G = 2048); from 4096 rows on the two run level or the
  // 8-wave kernel leads.
  if (a.s.G <= 2048) return launch_fwd_t<D, 4, 1, ROPE>(a, rope, stream);
  return launch_fwd_pp<D, ROPE>(a, rope, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, const RopeTable* rope, hipStream_t stream) {
  const bool r = rope != nullptr;
  if (a.s.D == 64) return r ? launch_fwd_d<64, true>(a, rope, stream) : launch_fwd_d<64, false>(a, rope, stream);
  return r ? launch_fwd_d<128, true>(a, rope, stream) : launch_fwd_d<128, false>(a, rope, stream);
}

}  // namespace s2a
