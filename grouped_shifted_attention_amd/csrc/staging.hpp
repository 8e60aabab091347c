// Global -> LDS staging of bf16 row tiles for the S2-Attn kernels, and the
// LDS read helpers that turn them into MFMA operands.
//
// A tile is R rows x D columns of a [rows, heads, D] tensor whose rows are
// gathered through the roll/group index map.  Tiles are loaded ahead of use,
// straight into LDS, so global latency hides behind MFMA work.
//
// LDS layout: row-major with one padding chunk (16 bytes) after every row,
// i.e. a row stride of D + 8 elements, so successive rows start one bank
// group (16 bytes = 4 of the 64 four-byte banks) further on.  Two read
// shapes must be free of bank conflicts:
//   row read (16 bytes per lane, 16 lanes per cycle): 16 tile rows, one
//     chunk each -- conflict-free for any 16 rows distinct mod 16;
//   transposing read (8 bytes per lane, 32 lanes per cycle): 4 tile rows x
//     4 consecutive chunks x 2 halves -- conflict-free when the 4 rows are
//     4 apart.
// Both hold because each 16-row block of a tile is visited in the order
//   rowperm(m) = 4*(m%4) + 2*(m/8) + (m/4)%2   (an involution),
// i.e. MFMA operand row m of a 16-row block is tile row rowperm(m).  The
// rows a C accumulator hands a lane (8*(r/4) + 4*hh + r%4, the reduction
// order when that C tile is fed back as a B operand) then map to tile rows
// 4*t + hh (elements 0-3) and 4*t + 2 + hh (elements 4-7): 4 apart, as the
// transposing read wants.  All addresses stay a per-lane base plus
// compile-time offsets.
#pragma once

#include "device_common.hpp"

namespace s2a {

// Tile row of MFMA operand row m (0..31) of a 32-row block.
__device__ __forceinline__ constexpr int rowperm32(int m) {
  return (m & 16) | (((m & 3) << 2) | (((m >> 3) & 1) << 1) | ((m >> 2) & 1));
}
// Tile row of accumulator element r (0..15) of a lane in half hh of a
// 32 x 32 C tile whose rows were produced from rowperm32-ordered operands.
__device__ __forceinline__ constexpr int acc_row(int r, int hh) { return rowperm32(8 * (r >> 2) + 4 * hh + (r & 3)); }

// Direct global -> LDS staging (global_load_lds_dwordx4) of an R x D tile
// into the padded layout; no VGPRs hold the data.  One wave instruction
// moves 64 lanes x 16 bytes into 1 KB of LDS, lane l's bytes at +16*l, so
// instruction `inst` fills slots 64*inst .. 64*inst+63 of the tile, slot q
// being chunk q % (D/8 + 1) of row q / (D/8 + 1).  Lanes on a padding slot,
// or past the last row, fetch a harmless in-bounds chunk (row clamped, chunk
// 0) into LDS that is never read, so every lane of every instruction loads.
// The NW waves of the workgroup split the instructions round-robin.
// Completion is tracked by vmcnt: wait (s_waitcnt vmcnt) and barrier before
// the tile is read.
template <int D, int R, int NW>
struct LdsStage {
  static constexpr int CH = D / 8;
  static constexpr int RS = D + 8;               // LDS row stride (elements)
  static constexpr int SLOTS = R * (CH + 1);
  static constexpr int INSTR = (SLOTS + 63) / 64;
  static constexpr int ELEMS = INSTR * 512;      // LDS elements a tile occupies
  static constexpr int PER = (INSTR + NW - 1) / NW;
  int off[PER];  // fast path: element offset of the lane's chunk in a contiguous tile

  __device__ __forceinline__ static int slot_row(int inst, int lane) {
    return min((inst * 64 + lane) / (CH + 1), R - 1);
  }
  __device__ __forceinline__ static int slot_col(int inst, int lane) {
    const int q = inst * 64 + lane;
    const int c = q % (CH + 1);
    return (q < SLOTS && c < CH) ? c << 3 : 0;
  }

  __device__ __forceinline__ LdsStage(int wave, int lane, int row_stride) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int inst = wave + k * NW;
      off[k] = slot_row(inst, lane) * row_stride + slot_col(inst, lane);
    }
  }

  // Wave-instructions this wave issues per tile (wave-uniform).
  __device__ __forceinline__ static int count(int wave) {
    return INSTR % NW == 0 ? PER : (INSTR - wave + NW - 1) / NW;
  }

  __device__ __forceinline__ static void dma(const uint16_t* src, uint16_t* dst) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
  }

  // R consecutive rows starting at `tile0` (see contig_tile).
  __device__ __forceinline__ void load_contig(const uint16_t* tile0, uint16_t* lds, int wave) const {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int inst = wave + k * NW;
      if (INSTR % NW == 0 || inst < INSTR) dma(tile0 + off[k], lds + inst * 512);
    }
  }

  // General rows: `row_ptr(r)` must return a readable row for every r < R
  // (callers point rows past the group end at a valid row; those rows only
  // ever meet exact-zero weights).
  template <class RowPtr>
  __device__ __forceinline__ void load_rows(RowPtr row_ptr, uint16_t* lds, int wave, int lane) const {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int inst = wave + k * NW;
      if (INSTR % NW == 0 || inst < INSTR)
        dma(row_ptr(slot_row(inst, lane)) + slot_col(inst, lane), lds + inst * 512);
    }
  }
};

// Direct global -> LDS load of 4 bytes per lane: lane l's word lands at
// dst + 4*l bytes (dst is wave-uniform).
__device__ __forceinline__ void dma4(const float* src, float* dst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)dst, 4, 0, 0);
}

// s_waitcnt on vmcnt only: wait until at most N of this wave's global loads
// (LDS DMA included) are outstanding.  gfx9 immediate: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4 and lgkmcnt 11:8 set to their maxima (no wait).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | 0x70 | 0xF00);
}

__device__ __forceinline__ void wait_vmem_all() { wait_vmcnt<0>(); }

// Workgroup barrier for LDS hand-overs: completes this wave's LDS accesses
// (lgkmcnt) and meets the other waves.  Unlike __syncthreads() it does not
// drain outstanding global loads (a workgroup fence waits for them, direct-
// to-LDS loads included), so loads of later tiles stay in flight across it;
// callers first wait (vmcnt) for the tile the next step reads.  The "memory"
// clobber keeps the compiler from moving memory accesses across it.
#ifdef S2A_DEBUG_BARRIERS
// Race-check build: every LDS hand-over drains all outstanding memory
// operations (global loads and direct-to-LDS loads included) and meets a full
// workgroup barrier.  Its results must equal the normal build's bit for bit;
// a difference exposes a hand-over that relies on a missing wait or barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}
#else
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
#endif

// wait_vmcnt for a wave-uniform count known only at run time (0..16; larger
// counts wait for everything, which is always safe).
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  switch (n) {
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    case 15: wait_vmcnt<15>(); break;
    case 16: wait_vmcnt<16>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

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

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i supplies 4
// consecutive 16-bit elements M[4i..4i+3]; lane j receives M[j], M[16+j],
// M[32+j], M[48+j].  Four lanes pointing at 4 consecutive columns of one row
// thus form one row of a 4 x 16 block, and every lane receives one column of
// it across the 4 rows.
__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// Per-lane addressing of the padded tiles, computed once per kernel.
//
// Row read (MFMA operand with k = d): operand row m = lane%32 of a 32-row
// block at tile row rb (a multiple of 32) is tile row rb + rowperm32(m);
// k-step kk covers chunk 2*kk + lane/32.
//
// Transposed read (MFMA A operand with k = tile row): lane l belongs to group
// g = l/16 (hh = g/2 picks the C-order half, g%2 the 16-column half) and has
// i = l%16.  Lanes 4t..4t+3 of a group supply 4-column pieces of one tile
// row, which the instruction hands out so that every lane receives one
// column across the group's 4 rows.  For the 16-row block at k0 (a multiple
// of 16) the lo read covers rows k0 + 4t + hh, the hi read rows
// k0 + 4t + 2 + hh (t = 0..3), which are the tile rows of accumulator
// elements 0-3 and 4-7 (see acc_row); the lane's column is 32*db + lane%32.
template <int D>
struct TileLane {
  static constexpr int RS = D + 8;
  int rbase;  // row read: element offset of the lane's row and chunk
  int tbase;  // transposed read: element offset of the lane's lo row piece

  __device__ __forceinline__ explicit TileLane(int lane) {
    const int l32 = lane & 31, hh = lane >> 5;
    rbase = rowperm32(l32) * RS + hh * 8;
    const int g = lane >> 4, i = lane & 15;
    tbase = (4 * (i >> 2) + (g >> 1)) * RS + (2 * (g & 1) + ((i & 3) >> 1)) * 8 + 4 * (i & 1);
  }

  __device__ __forceinline__ bf16x8 row(const uint16_t* tile, int rb, int kk) const {
    return lds_frag(tile + rb * RS + rbase + 16 * kk);
  }

  __device__ __forceinline__ bf16x8 tr(const uint16_t* tile, int k0, int db) const {
    const uint16_t* p = tile + k0 * RS + tbase + 32 * db;
    const s16x4 lo = lds_read_tr(p);
    const s16x4 hi = lds_read_tr(p + 2 * RS);
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
};

}  // namespace s2a
