// Global -> VGPR -> LDS staging of bf16 row tiles for the S2-Attn kernels.
//
// A tile is R rows x D columns of a [rows, heads, D] tensor whose rows are
// gathered through the roll/group index map (the caller's `addr(row)`
// returns the row's global address, or nullptr for rows past the group end,
// which are staged as zeros).  Loads are issued one tile ahead (into VGPRs)
// and written to LDS after the current tile's math, so global latency hides
// behind MFMA work.
//
// Two LDS layouts:
//   row-major   [R][D + 8]     rows are MFMA A operands with k = d
//                              (16-byte reads; the 16-byte pad spreads the
//                              rows of one read over the banks)
//   transposed  [D][R + 8]     rows are MFMA A operands with k = tile row;
//                              inside every 16-row block the rows sit in the
//                              order tr_slot() gives, which matches the rows
//                              a C accumulator hands each lane (see
//                              device_common.hpp), so one 16-byte read per
//                              lane fetches a whole k-slice.
#pragma once

#include "device_common.hpp"

namespace s2a {

// Row-major copy.  Items are 16-byte chunks, chunk index fastest, so a wave's
// global loads are contiguous row segments and its LDS writes hit distinct
// banks.
template <int D, int R, int NT>
struct RowStage {
  static constexpr int CH = D / 8;
  static constexpr int ITEMS = R * CH;
  static constexpr int PER = (ITEMS + NT - 1) / NT;
  static constexpr int STR = D + 8;
  u32x4 r[PER];

  template <class Addr>
  __device__ __forceinline__ void load(int tid, Addr addr) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int item = tid + i * NT;
      if (ITEMS % NT == 0 || item < ITEMS) {
        const int row = item / CH, ch = item % CH;
        const uint16_t* p = addr(row);
        r[i] = p ? ld16(p + ch * 8) : zero_u4();
      }
    }
  }

  // Fast path: the R rows are consecutive rows of the tensor starting at
  // `tile0` (no group end, no wrap inside the tile), `row_stride` elements
  // apart.  The per-thread offset is loop-invariant, so each load is one
  // instruction off a uniform base.
  __device__ __forceinline__ void load_contig(int tid, const uint16_t* tile0, int row_stride) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int item = tid + i * NT;
      if (ITEMS % NT == 0 || item < ITEMS) {
        const int row = item / CH, ch = item % CH;
        r[i] = ld16(tile0 + (row * row_stride + ch * 8));
      }
    }
  }

  __device__ __forceinline__ void store(int tid, uint16_t* lds) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int item = tid + i * NT;
      if (ITEMS % NT == 0 || item < ITEMS) {
        const int row = item / CH, ch = item % CH;
        *reinterpret_cast<u32x4*>(lds + row * STR + ch * 8) = r[i];
      }
    }
  }
};

// Quad copy: items are (4-row quad, 8-column octet) blocks, quad index
// fastest.  Feeds the transposed layout (each thread owns 4 rows x 8 columns
// and writes 8 columns x 4 rows as 8-byte words, the quads of one wave
// landing in distinct banks) and optionally the row-major layout too.
template <int D, int R, int NT>
struct QuadStage {
  static constexpr int CH = D / 8;
  static constexpr int NQ = R / 4;
  static constexpr int ITEMS = NQ * CH;
  static constexpr int PER = (ITEMS + NT - 1) / NT;
  static constexpr int STR = D + 8;
  static constexpr int TSTR = R + 8;
  u32x4 r[PER][4];

  template <class Addr>
  __device__ __forceinline__ void load(int tid, Addr addr) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int item = tid + i * NT;
      if (ITEMS % NT == 0 || item < ITEMS) {
        const int rq = item % NQ, oc = item / NQ;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint16_t* p = addr(rq * 4 + u);
          r[i][u] = p ? ld16(p + oc * 8) : zero_u4();
        }
      }
    }
  }

  // Fast path for R consecutive rows starting at `tile0` (see RowStage).
  __device__ __forceinline__ void load_contig(int tid, const uint16_t* tile0, int row_stride) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int item = tid + i * NT;
      if (ITEMS % NT == 0 || item < ITEMS) {
        const int rq = item % NQ, oc = item / NQ;
        const int off = rq * 4 * row_stride + oc * 8;
#pragma unroll
        for (int u = 0; u < 4; ++u) r[i][u] = ld16(tile0 + u * row_stride + off);
      }
    }
  }

  // row_lds may be nullptr (transposed copy only).
  __device__ __forceinline__ void store(int tid, uint16_t* row_lds, uint16_t* tr_lds) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int item = tid + i * NT;
      if (ITEMS % NT == 0 || item < ITEMS) {
        const int rq = item % NQ, oc = item / NQ;
        if (row_lds != nullptr) {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            *reinterpret_cast<u32x4*>(row_lds + (rq * 4 + u) * STR + oc * 8) = r[i][u];
        }
        const int pos = (rq >> 2) * 16 + tr_slot((rq & 3) * 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          u32x2 pr;
          if (e & 1) {
            pr[0] = pack_hi(r[i][0][w], r[i][1][w]);
            pr[1] = pack_hi(r[i][2][w], r[i][3][w]);
          } else {
            pr[0] = pack_lo(r[i][0][w], r[i][1][w]);
            pr[1] = pack_lo(r[i][2][w], r[i][3][w]);
          }
          *reinterpret_cast<u32x2*>(tr_lds + (oc * 8 + e) * TSTR + pos) = pr;
        }
      }
    }
  }
};

// Start of a tile of R local rows beginning at local row j0 of a group whose
// first rolled row is at original position `base`, if those R rows are R
// consecutive original positions inside the group; nullptr otherwise (the
// tile reaches past the group end or wraps around the sequence end).
__device__ __forceinline__ const uint16_t* contig_tile(const uint16_t* head0, long long row_stride, int base,
                                                       int j0, int R, int G, int N) {
  if (j0 + R > G) return nullptr;
  const int p0 = base + j0;
  if (p0 < N && p0 + R > N) return nullptr;
  return head0 + (long long)(p0 >= N ? p0 - N : p0) * row_stride;
}

// 16-byte LDS read as an MFMA operand.
__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* p) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(p));
}

}  // namespace s2a
