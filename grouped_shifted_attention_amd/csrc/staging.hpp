// Global -> LDS staging of bf16 row tiles for the S2-Attn kernels, and the
// LDS read helpers that turn them into MFMA operands.
//
// A tile is R rows x D columns of a [rows, heads, D] tensor whose rows are
// gathered through the roll/group index map.  Tiles are loaded one step
// ahead, straight into LDS, so global latency hides behind MFMA work.
//
// LDS layout: row-major [R][D] with the 16-byte chunks of each row XOR-
// swizzled: logical chunk c of row r is stored at chunk c ^ swz(r),
// swz(r) = 2*(r & 3) + ((r >> 2) & 1).  A row is an MFMA operand with k = d
// (one 16-byte read per lane, 8 consecutive rows per read pass); a column
// block is an MFMA operand with k = row through the transposing LDS read
// (4 consecutive rows x 32 bytes per 16 lanes).  The swizzle puts both read
// shapes, and the row writes, on distinct banks; no single row padding can.
#pragma once

#include "device_common.hpp"

namespace s2a {

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

// Direct global -> LDS staging (global_load_lds_dwordx4) of an R x D tile
// into the swizzled layout; no VGPRs hold the data.  One wave instruction
// moves 64 lanes x 16 bytes into 1 KB of LDS, lane l's bytes at +16*l, so
// instruction `inst` fills tile chunks 64*inst .. 64*inst+63, i.e. physical
// chunk p = q % (D/8) of row q / (D/8); the lane fetches the logical chunk
// p ^ swz(row) from global memory.  The NW waves of the workgroup split the
// R*D/512 instructions round-robin.  Completion is tracked by vmcnt: wait
// (s_waitcnt vmcnt) and barrier before the tile is read.
template <int D, int R, int NW>
struct LdsStage {
  static constexpr int CH = D / 8;
  static constexpr int INSTR = R * CH / 64;
  static constexpr int PER = (INSTR + NW - 1) / NW;
  static_assert(R * CH % 64 == 0, "tile must be a whole number of 1 KB wave loads");
  int off[PER];  // fast path: element offset of the lane's chunk in a contiguous tile

  __device__ __forceinline__ static int chunk_row(int inst, int lane) { return (inst * 64 + lane) / CH; }
  __device__ __forceinline__ static int chunk_col(int inst, int lane) {
    const int q = inst * 64 + lane;
    return ((q % CH) ^ swz(q / CH)) << 3;
  }

  __device__ __forceinline__ LdsStage(int wave, int lane, int row_stride) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int inst = wave + k * NW;
      off[k] = chunk_row(inst, lane) * row_stride + chunk_col(inst, lane);
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
        dma(row_ptr(chunk_row(inst, lane)) + chunk_col(inst, lane), lds + inst * 512);
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
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// wait_vmcnt for a wave-uniform count known only at run time (0..8).
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

// Per-lane addressing of the swizzled tiles, computed once per kernel.
//
// Row read (MFMA operand with k = d): the lane's row is rb + lane%32 (rb a
// multiple of 8), k-step kk covers logical chunk 2*kk + lane/32.  Because
// swz() only touches the low 3 chunk bits and depends only on row % 8, the
// offset is rb*D + 64*(kk/4) + row_off[kk%4].
//
// Transposed read (MFMA A operand with k = tile row): lane l belongs to group
// g = l/16 (hh = g/2 picks the row half, g%2 the 16-column half) and has
// i = l%16 (row i/4 of a 4-row block, 4-element column chunk i%4).  Element
// s of a lane in half hh is row k0 + 8*(s/4) + 4*hh + s%4 (the order a C
// accumulator hands a lane its rows) and its column is 32*db + lane%32; the
// offset is k0*D + 64*(db/2) + tr_off[db%2] (+ 8*D for the second 4 rows).
template <int D>
struct SwzLane {
  int row_off[4];
  int tr_off[2];

  __device__ __forceinline__ explicit SwzLane(int lane) {
    const int l32 = lane & 31, hh = lane >> 5;
    const int y = hh ^ swz(l32 & 7);
#pragma unroll
    for (int q = 0; q < 4; ++q) row_off[q] = l32 * D + (((2 * q) ^ y) << 3);
    const int g = lane >> 4, i = lane & 15;
    const int r = 4 * (g >> 1) + (i >> 2);
    const int lc = 2 * (g & 1) + ((i & 3) >> 1);
#pragma unroll
    for (int od = 0; od < 2; ++od) tr_off[od] = r * D + (((4 * od + lc) ^ swz(r)) << 3) + 4 * (i & 1);
  }

  __device__ __forceinline__ bf16x8 row(const uint16_t* tile, int rb, int kk) const {
    return lds_frag(tile + rb * D + ((kk >> 2) << 6) + row_off[kk & 3]);
  }

  __device__ __forceinline__ bf16x8 tr(const uint16_t* tile, int k0, int db) const {
    const uint16_t* p = tile + k0 * D + ((db >> 1) << 6) + tr_off[db & 1];
    const s16x4 lo = lds_read_tr(p);
    const s16x4 hi = lds_read_tr(p + 8 * D);  // swz(r + 8) == swz(r)
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
};

}  // namespace s2a
