// gla_records.h -- the per-chunk records that the forward's prep pass writes
// and its recurrence pass streams through LDS: their fragment-blocked unit
// orders and sizes.
#pragma once

#include "gla_common.h"

namespace gla {

// ---- fragment-blocked layouts ---------------------------------------------
// chunk_prep writes each chunk's Q~, K~, P (and P's diagonal low parts) as
// blocks of 16-byte units laid out the way the recurrence's MFMA operand
// reads want them, so that chunk_recur stages a chunk with contiguous
// 1 KB copies and reads every operand at a lane-constant LDS offset.  The
// unit orders below are involutions (applying one twice gives the identity),
// chosen so that each operand read is free of LDS bank conflicts (64 banks of
// 4 bytes; one 256-byte bank span per pass).
//
// Row block (Q~, P): 16 rows x 4 units.  A 16x16 MFMA operand read has lane
// (g, n) load unit g of row n; the 16 lanes of one g then cover 16 distinct
// units of a 256-byte span.
__device__ inline int row_slot(int n, int g) { return n * 4 + (g ^ ((n >> 2) & 3)); }
// Diagonal-block low part (bf16): 16 rows x 2 units (columns 0-7, 8-15).
__device__ inline int lo_slot(int n, int gd) { return n * 2 + (gd ^ ((n >> 3) & 1)); }
// Token-run block (bf16, transposed reads): 32 rows x UPR units.  A
// ds_read_b64_tr_b16 operand read touches rows 8 g + j (+ 4), j < 4, 32 bytes
// each; half a wave (g = 0, 1) then covers 8 distinct 32-byte windows.
template <int UPR>
__device__ inline int run_slot(int rho, int u) {
  int m;
  if constexpr (UPR == 2) m = ((rho >> 3) & 1) << 3;
  else if constexpr (UPR == 4) m = ((rho >> 3) & 1) << 1;
  else m = (((rho >> 1) & 1) | (((rho >> 3) & 1) << 1)) << 1;
  return (rho * UPR + u) ^ m;
}
// Scalar-read block (fp32): 16 rows x UPR units.  A 16x16x4 operand read has
// lane group g read row 4 g + i (fixed i), 64 bytes; the XOR puts the four
// rows in distinct 64-byte windows of a 256-byte span.
template <int UPR>
__device__ inline int scal_slot(int rho, int u) { return (rho * UPR + u) ^ (((rho >> 2) & 3) << 2); }

// Per-chunk record sizes (bytes).  GW: elements per 64-byte column group
// (one unit of 4 per row of a row block).
template <typename T>
struct RecDims {
  static constexpr int ES = (int)sizeof(T);
  static constexpr bool BF = ES == 2;
  static constexpr int EPU = 16 / ES;
  static constexpr int GW = 64 / ES;
  __host__ __device__ static constexpr int gbytes(int dk) { return ((8 * dk + 1023) / 1024) * 1024; }
  // P's row block jt (16 rows) holds column groups 0 .. plast(jt); the
  // groups after it lie above the diagonal and are not stored.  pblock: the
  // 1 KB block (jt, cg) in the packed record; pblocks: blocks per chunk.
  __host__ __device__ static constexpr int plast(int jt) { return (16 * jt + 15) / GW; }
  __host__ __device__ static constexpr int pblock(int jt, int cg) {
    static_assert(GW == 32 || GW == 16, "bf16 or fp32 records");
    // sum over j < jt of plast(j) + 1: j / 2 + 1 (GW 32) or j + 1 (GW 16)
    return (GW == 32 ? jt + ((jt - 1) >> 1) * (jt >> 1) : jt * (jt + 1) / 2) + cg;
  }
  __host__ __device__ static constexpr int pblocks(int C) { return pblock(C / 16, 0); }
};

constexpr int kLdsLimit = 160 * 1024;

}  // namespace gla
