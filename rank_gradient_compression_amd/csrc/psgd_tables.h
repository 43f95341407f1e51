// Device tables of a compression plan: the layout the host plan writes into
// the workspace and the kernels read.  Plain structs, shared by the host-only
// plan code and the HIP kernels of this library.
#pragma once

#include <stdint.h>

namespace psgd {

// Rows of a compressed matrix handled by one wavefront in the streaming
// passes (EF-add + P = M Q, the residual pass and decompression), and the
// wavefronts of one workgroup.  A workgroup covers kWaveRows * kWavesPerWG
// consecutive rows of one matrix, every column.
constexpr int kWaveRows = 8;
constexpr int kWavesPerWG = 4;
constexpr int kWGThreads = 64 * kWavesPerWG;
constexpr int kRowsPerWG = kWaveRows * kWavesPerWG;

// Columns of one M^T P_hat workgroup tile per 4-wide vector lane: each of the
// four wavefronts owns 64 lanes * vec columns.
constexpr int kMtpWaves = 4;

// Largest rank the VALU streaming kernels handle; larger ranks use the MFMA
// kernels.
constexpr int kValuMaxRank = 8;

// Columns a compressed matrix may have (exclusive): the streaming kernels
// address a row from a wavefront-uniform base with a 32-bit byte offset.
constexpr int64_t kMaxCols = int64_t(1) << 30;

// Alignment (elements) of every region the plan lays out.
constexpr int64_t kAlignElems = 64;

// Tiles of the MFMA kernels (ranks above kValuMaxRank, padded to a multiple
// of 16).
constexpr int kMfmaRows = 64;      // rows of one MFMA pass-1 / pass-3 workgroup tile
constexpr int kMfmaCols = 128;     // columns of one MFMA pass-2 workgroup tile
constexpr int kGramRows = 128;     // rows of one Gram-partial / apply workgroup

// One compressed matrix.
struct MatDesc {
  int64_t off;       // flat element offset of row 0 in grads/err/mom/mhat
  int64_t p_off;     // P / P_hat: rank columns of m floats from here
  int64_t q_off;     // Q: rank columns of n floats from here
  int64_t part_off;  // partial-Q scratch (floats, from the scratch base)
  int64_t gram_off;  // Gram partials (doubles, from the Gram scratch base)
  int64_t ppart_off; // partial-P scratch of a column-split pass 1 (elements: fp32
                     // on the vector path, fp64 on the matrix cores)
  int64_t t_off;     // triangular factor T (doubles, from the Gram scratch base)
  int32_t m, n;
  int32_t vec;       // 4, 2 or 1: widest vector access both n and off allow
  int32_t nrb;       // row blocks of the M^T P_hat pass
  int32_t rb_rows;   // rows per row block of the M^T P_hat pass
  int32_t ncb;       // column tiles of the M^T P_hat pass
  int32_t wg_rows0;  // first workgroup of this matrix in the pass-1 row-tile grid
  int32_t wg_mtp0;   // first workgroup of this matrix in the M^T P_hat grid
  int32_t wg_red0;   // first workgroup of this matrix in the Q-reduce grid
  int32_t s1;        // pass 1: column splits
  int32_t s1_cols;   // pass 1: columns per split (whole wavefront widths)
  int32_t wg_pred0;  // first workgroup in the P-partial reduce grid (s1 > 1)
  int32_t wg_gram0;  // first workgroup in the Gram-partial / apply grid
  int32_t ngb;       // Gram-partial blocks (kGramRows rows each)
  int32_t tensor;    // index of the tensor in the plan
  int32_t red_split; // wavefronts summing one 64-element slice of Q partials
  int32_t s3;        // residual / decompression pass: column splits; 0: the
                     // vector path tiles the matrix flat (psgd_flat.h)
  int32_t s3_cols;   // residual / decompression pass: columns per split
                     // (with s3 == 0: elements per workgroup)
  int32_t wg_rec0;   // first workgroup of this matrix in the residual-pass grid
  int32_t pad_[3];
};
static_assert(sizeof(MatDesc) == 144, "MatDesc layout");

// One pass-through tensor: `len` elements at flat offset `off`, packed at
// `p_off` (absolute, in the P buffer).
struct PassDesc {
  int64_t off;
  int64_t p_off;
  int64_t len;
  int64_t wg0;  // first workgroup of this tensor in the pass-through grid
};

// One factor to orthonormalise (P of a matrix, or Q / P inside the refresh):
// `rows` x rank, column-major with leading dimension `rows`, from element
// `off` of the buffer given at launch.
struct OrthDesc {
  int64_t off;
  int64_t gram_off;  // Gram partials (doubles, from the Gram scratch base)
  int64_t t_off;     // triangular factor T (doubles)
  int32_t rows;
  int32_t ngb;       // Gram-partial blocks of kGramRows rows
  int32_t wg0;       // first workgroup in the grouped Gram grid
  int32_t pad_;
};

constexpr int kPassChunk = 4096;  // elements per pass-through workgroup
constexpr int kRedCols = 256;     // P elements per column-split reduce workgroup
constexpr int kRedWaves = 16;     // wavefronts of one Q-reduce workgroup

// Row-tile workgroups passes 1 and 3 aim for (the columns are split until the
// grid has this many).
constexpr int kRowTilesTarget = 1024;

// Column splits of passes 1 and 3.  A workgroup streams a few rows of its
// split, so the split width sets how much of each array it touches at once.
// On the vector path pass 1 (two arrays read, one written, plus the P row
// sums at the end) and the residual pass (one read, two written) both take
// one 256-column piece per wavefront row: a workgroup is one 32-row x
// 256-column tile, and the grid's dispatch order walks the arrays as one
// contiguous front (1024-column pass-1 splits were 10% slower on the 7B-shaped
// set once its loads and stores stream).  The matrix-core pass 1 keeps
// kEfpSplitColsMfma-column splits (narrower, down to 256 columns, while the
// grid is short of kRowTilesTarget workgroups): its column-split partials of
// P are r fp64 values per row and split.
constexpr int kEfpSplitCols = 256;
constexpr int kEfpSplitColsMfma = 1024;
constexpr int kRecSplitCols = 256;

// Header at the start of the workspace.
struct WsHeader {
  uint64_t magic;
  int32_t nmat, npass;
  int32_t rank, flags;
  int32_t wg_rows, wg_mtp, wg_red, wg_pass;
  int32_t wg_pred, wg_gram, wg_gramq, rank_pad, mfma, wg_rec;
  int32_t wg_rows_v4;    // matrix cores: pass-1 workgroups of the 16-byte-row matrices (first)
  int32_t pad_;
  int64_t mat_off;       // bytes from workspace start: MatDesc[nmat]
  int64_t pass_off;      // PassDesc[npass]
  int64_t rows_map_off;  // int32 matrix index per row-tile workgroup (pass 1)
  int64_t rec_map_off;   // int32 matrix index per residual-pass workgroup
  int64_t mtp_map_off;   // int32 per M^T P_hat workgroup
  int64_t red_map_off;   // int32 per Q-reduce workgroup
  int64_t pass_map_off;  // int32 pass-through tensor per pass-through workgroup
  int64_t pred_map_off;  // int32 per P-partial reduce workgroup
  int64_t gram_map_off;  // int32 per Gram-partial / apply workgroup
  int64_t gramq_map_off; // int32 per Gram workgroup over the Q factors (refresh)
  int64_t orth_off;      // OrthDesc[3 * nmat]: P of compress, refresh P, refresh Q
  int64_t tables_bytes;  // bytes of the table part (uploaded by workspace_init)
  int64_t part_base;     // bytes: partial-Q scratch (float)
  int64_t ppart_base;    // bytes: partial-P scratch (float; double on the matrix cores)
  int64_t gram_base;     // bytes: orthonormalisation scratch (double)
  int64_t refresh_base;  // bytes: refresh scratch (float)
  int64_t total_bytes;
};

constexpr uint64_t kWsMagic = 0x3144474953505350ull;  // "PSPSIGD1"

}  // namespace psgd
