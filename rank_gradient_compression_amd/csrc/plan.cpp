// Host-only compression plan: classification of a model's tensors, the packed
// layout of the factors and the workgroup tile tables the kernels consume.
// Nothing here touches a device.
//
// Classification follows the "Method" section of the anthology note on
// PowerSGD (note 152): each layer's gradient is approximated independently,
// conv tensors viewed as matrices, bias vectors and small tensors sent
// uncompressed.  "Small" is read as r*(m+n) >= m*n, i.e. the factors would not
// be smaller than the matrix (the glossary entry "PowerSGD" gives the payload
// as O(r(m+n)) instead of O(mn)).

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <new>
#include <numeric>

#include "psgd_flat.h"
#include "psgd_internal.h"

namespace psgd {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
}

void clear_error() { g_err[0] = 0; }

static std::atomic<uint64_t> g_next_plan_id{1};

static int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Rows per row block of the M^T P_hat pass.  The row-block partial sums cost
// 2*rank/rb_rows of that pass's matrix traffic, so a block has at least
// 8*rank rows (at most 1/4 extra on the pass; 16*rank up to 512 rows on the
// matrix cores); above that, blocks are as long as possible while the grid
// still has enough workgroups to cover the chip.
static int32_t choose_rb_rows(const std::vector<MatDesc>& mats, int64_t rank, bool mfma) {
  const int64_t target_wgs = 2048;
  int32_t rb_min = 64;
  // matrix cores: a block of rb rows writes r partial values per column for
  // the rb it reads, so blocks take at least 16 r rows, capped at 512: the
  // partials stay within 1/16 of the pass's reads up to rank 32 and 1/8 at
  // rank 64
  const int64_t want = mfma ? std::min<int64_t>(16 * rank, 512) : 8 * rank;
  while (rb_min < want) rb_min *= 2;
  int32_t rb = 2048;
  for (; rb > rb_min; rb /= 2) {
    int64_t wgs = 0;
    for (const MatDesc& d : mats) {
      const int64_t cols_per_wg = mfma ? kMfmaCols : (int64_t)kMtpWaves * 64 * d.vec;
      wgs += ((d.m + rb - 1) / rb) * ((d.n + cols_per_wg - 1) / cols_per_wg);
    }
    if (wgs >= target_wgs) break;
  }
  return rb;
}

}  // namespace psgd

using namespace psgd;

extern "C" psgd_status_t psgd_plan_create(int32_t ntensors, const int64_t* rows, const int64_t* cols,
                                          const int64_t* offsets, int32_t rank, uint32_t flags,
                                          float beta, psgd_plan_t* out) {
  clear_error();
  if (!out) {
    set_error("psgd_plan_create: out is NULL");
    return PSGD_ERR_INVALID_ARG;
  }
  *out = nullptr;
  if (ntensors < 0 || (ntensors > 0 && (!rows || !cols))) {
    set_error("psgd_plan_create: bad tensor list (ntensors=%d)", ntensors);
    return PSGD_ERR_INVALID_ARG;
  }
  if (rank < 1) {
    set_error("psgd_plan_create: rank %d < 1", rank);
    return PSGD_ERR_INVALID_ARG;
  }
  if (rank > PSGD_MAX_RANK) {
    set_error("psgd_plan_create: rank %d above the supported maximum %d", rank, PSGD_MAX_RANK);
    return PSGD_ERR_UNSUPPORTED;
  }
  if (flags & ~(PSGD_FLAG_MOMENTUM | PSGD_FLAG_GRADS_BF16)) {
    set_error("psgd_plan_create: unknown flag bits 0x%x", flags & ~(PSGD_FLAG_MOMENTUM | PSGD_FLAG_GRADS_BF16));
    return PSGD_ERR_UNSUPPORTED;
  }
  if ((flags & PSGD_FLAG_MOMENTUM) && !(beta == beta)) {
    set_error("psgd_plan_create: momentum beta is NaN");
    return PSGD_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < ntensors; ++i) {
    if (rows[i] < 1 || cols[i] < 0 || rows[i] > (int64_t)INT32_MAX || cols[i] > (int64_t)INT32_MAX) {
      set_error("psgd_plan_create: tensor %d has bad shape %lld x %lld", i, (long long)rows[i],
                (long long)cols[i]);
      return PSGD_ERR_INVALID_ARG;
    }
  }

  psgd_plan* p = new (std::nothrow) psgd_plan();
  if (!p) {
    set_error("psgd_plan_create: out of host memory");
    return PSGD_ERR_INVALID_ARG;
  }
  p->id = g_next_plan_id.fetch_add(1);
  p->ntensors = ntensors;
  p->rank = rank;
  p->flags = flags;
  p->beta = beta;
  p->rows.assign(rows, rows + ntensors);
  p->cols.resize(ntensors);
  p->numel.resize(ntensors);
  p->kind.resize(ntensors);
  p->flat_off.resize(ntensors);
  p->p_off.assign(ntensors, -1);
  p->q_off.assign(ntensors, -1);
  const int64_t r = rank;

  for (int32_t i = 0; i < ntensors; ++i) {
    const int64_t m = rows[i], n = cols[i] < 1 ? 1 : cols[i];
    p->cols[i] = n;
    p->numel[i] = m * n;
    if (cols[i] <= 1)
      p->kind[i] = PSGD_KIND_VECTOR;
    else
      p->kind[i] = (r * (m + n) < m * n) ? PSGD_KIND_COMPRESSED : PSGD_KIND_PASSTHRU;
    // the streaming kernels address a row with 32-bit byte offsets
    if (p->kind[i] == PSGD_KIND_COMPRESSED && n >= kMaxCols) {
      set_error("psgd_plan_create: tensor %d has %lld columns; a compressed matrix has fewer than %lld", i,
                (long long)n, (long long)kMaxCols);
      delete p;
      return PSGD_ERR_UNSUPPORTED;
    }
  }

  // Flat layout.
  if (offsets) {
    std::vector<int32_t> order(ntensors);
    std::iota(order.begin(), order.end(), 0);
    for (int32_t i = 0; i < ntensors; ++i) {
      if (offsets[i] < 0) {
        set_error("psgd_plan_create: tensor %d has negative offset", i);
        delete p;
        return PSGD_ERR_INVALID_ARG;
      }
    }
    std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return offsets[a] < offsets[b]; });
    int64_t end = 0;
    for (int32_t k = 0; k < ntensors; ++k) {
      const int32_t i = order[k];
      if (offsets[i] < end) {
        set_error("psgd_plan_create: tensor %d overlaps the previous tensor", i);
        delete p;
        return PSGD_ERR_INVALID_ARG;
      }
      end = offsets[i] + p->numel[i];
    }
    for (int32_t i = 0; i < ntensors; ++i) p->flat_off[i] = offsets[i];
    p->flat_elems = (size_t)end;
  } else {
    int64_t off = 0;
    for (int32_t i = 0; i < ntensors; ++i) {
      p->flat_off[i] = off;
      off = align_up(off + p->numel[i], kAlignElems);
    }
    p->flat_elems = (size_t)off;
  }

  // Packed factor layout: P_hat regions, then pass-through values; Q regions.
  int64_t poff = 0, qoff = 0;
  for (int32_t i = 0; i < ntensors; ++i) {
    if (p->kind[i] != PSGD_KIND_COMPRESSED) continue;
    const int64_t m = p->rows[i], n = p->cols[i];
    p->p_off[i] = poff;
    p->q_off[i] = qoff;
    poff = align_up(poff + r * m, kAlignElems);
    qoff = align_up(qoff + r * n, kAlignElems);
    p->payload += (size_t)(r * (m + n));
    p->dense += (size_t)(m * n);
    MatDesc d{};
    d.off = p->flat_off[i];
    d.p_off = p->p_off[i];
    d.q_off = p->q_off[i];
    d.m = (int32_t)m;
    d.n = (int32_t)n;
    d.tensor = i;
    d.vec = (n % 4 == 0 && d.off % 4 == 0) ? 4 : (n % 2 == 0 && d.off % 2 == 0) ? 2 : 1;
    p->mats.push_back(d);
    p->mat_tensor.push_back(i);
    p->max_m = std::max<int32_t>(p->max_m, (int32_t)m);
    p->max_n = std::max<int32_t>(p->max_n, (int32_t)n);
  }
  p->p_elems = (size_t)poff;
  p->q_elems = (size_t)qoff;
  int64_t ptoff = 0;
  for (int32_t i = 0; i < ntensors; ++i) {
    if (p->kind[i] == PSGD_KIND_COMPRESSED) continue;
    p->p_off[i] = poff + ptoff;
    PassDesc pd{};
    pd.off = p->flat_off[i];
    pd.p_off = poff + ptoff;
    pd.len = p->numel[i];
    p->pass.push_back(pd);
    ptoff = align_up(ptoff + p->numel[i], kAlignElems);
    p->payload += (size_t)p->numel[i];
  }
  p->pt_elems = (size_t)ptoff;

  // Tile tables.
  const bool mfma = rank > kValuMaxRank;
  const int64_t rp = align_up(r, 16);  // rank padding of the matrix-core and Gram kernels
  const int32_t rb = choose_rb_rows(p->mats, r, mfma);
  // Column splits of passes 1 and 3.  A wavefront streams a few rows of its
  // split, so the split width sets how much of each array a workgroup
  // touches at once: pass 1 in kEfpSplitCols-column pieces on the vector
  // path, kEfpSplitColsMfma on the matrix cores (halved, down to 256
  // columns, while the grid is short of kRowTilesTarget workgroups, as for a
  // set of few, short matrices), pass 3 in kRecSplitCols-column pieces.
  const int32_t tile_rows = mfma ? kMfmaRows : kRowsPerWG;
  int32_t w1 = mfma ? kEfpSplitColsMfma : kEfpSplitCols;
  for (;; w1 /= 2) {
    int64_t wgs = 0;
    for (const MatDesc& d : p->mats) {
      const int64_t cols = align_up(std::min<int64_t>(d.n, w1), mfma ? 64 : 64 * d.vec);
      wgs += ((d.m + tile_rows - 1) / tile_rows) * ((d.n + cols - 1) / cols);
    }
    if (wgs >= kRowTilesTarget || w1 <= 256) break;
  }
  int64_t part = 0, ppart = 0, gram = 0, rscr = 0;
  int32_t wg_rows = 0, wg_rec = 0, wg_mtp = 0, wg_red = 0, wg_pred = 0, wg_gram = 0;
  for (size_t k = 0; k < p->mats.size(); ++k) {
    MatDesc& d = p->mats[k];
    d.rb_rows = rb;
    d.nrb = (d.m + rb - 1) / rb;
    const int32_t cols_per_wg = mfma ? kMfmaCols : kMtpWaves * 64 * d.vec;
    d.ncb = (d.n + cols_per_wg - 1) / cols_per_wg;
    d.part_off = part;
    if (d.nrb > 1) part += align_up((int64_t)d.nrb * r * d.n, kAlignElems);
    // Q reduce: `red_split` wavefronts share one 64-element slice of Q, so
    // that each sums at most 8 row blocks (up to 16 wavefronts per slice).
    d.red_split = 1;
    while (d.red_split < kRedWaves && (d.nrb + d.red_split - 1) / d.red_split > 8) d.red_split *= 2;
    d.wg_rec0 = wg_rec;
    // column splits: a split is a whole number of wavefront widths (64
    // columns on the matrix cores, 64 vectors otherwise)
    const int32_t unit = mfma ? 64 : 64 * d.vec;
    d.s1_cols = (int32_t)align_up(std::min<int32_t>(d.n, w1), unit);
    d.s3_cols = (int32_t)align_up(std::min<int32_t>(d.n, kRecSplitCols), unit);
    d.s1 = (d.n + d.s1_cols - 1) / d.s1_cols;
    d.s3 = (d.n + d.s3_cols - 1) / d.s3_cols;
    // pass 1 tiles are kMfmaRows / kRowsPerWG rows; pass 3 tiles kRowsPerWG
    // rows on both paths
    const int32_t nrow_wg = ((d.m + tile_rows - 1) / tile_rows) * d.s1;
    int32_t nrec_wg = ((d.m + kRowsPerWG - 1) / kRowsPerWG) * d.s3;
    // Rows that do not start on 128-byte lines: the vector-path residual
    // pass tiles the matrix flat (s3 = 0, s3_cols elements per workgroup,
    // in pieces of kFlatChunk), with Q and the P_hat rows of the
    // workgroup's elements staged in LDS.
    const int64_t rq = flat_rq((int)r);
    if (!mfma && d.n % 32 != 0 && d.off % 32 == 0 && d.n >= kFlatMinCols && d.n * rq <= kFlatQMax &&
        (int64_t)d.m * d.n < (int64_t(1) << 31)) {
      // one staging of Q (n x rq floats) serves S pieces: one piece while Q
      // is at most a quarter of a piece's elements, up to kFlatSub (10000 x
      // 2046: pass 55.7 -> 51 us with four pieces; with four, the LSTM set's
      // short matrices had too few workgroups)
      const int64_t nsub = std::min<int64_t>(kFlatSub, std::max<int64_t>(1, d.n * rq / (kFlatChunk / 4)));
      const int64_t per_wg = (int64_t)kFlatChunk * nsub;
      d.s3 = 0;
      d.s3_cols = (int32_t)per_wg;
      nrec_wg = (int32_t)(((int64_t)d.m * d.n + per_wg - 1) / per_wg);
      const int64_t rows = per_wg / d.n + 2;  // rows one workgroup can touch
      p->flat_lds = std::max<size_t>(p->flat_lds, (size_t)((d.n + rows) * rq * sizeof(float)));
      static_assert(kFlatReconLdsMax <= 65536, "flat residual LDS bound");
    }
    d.ppart_off = ppart;
    d.wg_pred0 = wg_pred;
    if (d.s1 > 1) {
      ppart += align_up((int64_t)d.s1 * r * d.m, kAlignElems);
      const int32_t np = (int32_t)((r * d.m + kRedCols - 1) / kRedCols);
      for (int32_t t = 0; t < np; ++t) p->pred_map.push_back((int32_t)k);
      wg_pred += np;
    }
    p->nrow_wg.push_back(nrow_wg);
    for (int32_t t = 0; t < nrec_wg; ++t) p->rec_map.push_back((int32_t)k);
    wg_rec += nrec_wg;
    // Gram grid (orthonormalisation of P) and the Gram scratch, sized for P
    // (m rows) and for the refresh's Q (n rows)
    d.ngb = (d.m + kGramRows - 1) / kGramRows;
    d.wg_gram0 = wg_gram;
    for (int32_t t = 0; t < d.ngb; ++t) p->gram_map.push_back((int32_t)k);
    wg_gram += d.ngb;
    const int64_t nb = std::max<int64_t>(d.ngb, (d.n + kGramRows - 1) / kGramRows);
    d.gram_off = gram;
    d.t_off = gram + nb * rp * rp;
    gram += (nb + 1) * rp * rp;
    d.wg_mtp0 = wg_mtp;
    for (int32_t t = 0; t < d.nrb * d.ncb; ++t) p->mtp_map.push_back((int32_t)k);
    wg_mtp += d.nrb * d.ncb;
    d.wg_red0 = wg_red;
    if (d.nrb > 1) {
      const int32_t per_wg = 64 * (kRedWaves / d.red_split);
      const int32_t nred = (int32_t)((r * d.n + per_wg - 1) / per_wg);
      for (int32_t t = 0; t < nred; ++t) p->red_map.push_back((int32_t)k);
      wg_red += nred;
    }
    // refresh scratch: P of this matrix (rank columns of m rows)
    rscr = std::max<int64_t>(rscr, align_up((int64_t)d.m * rp, kAlignElems));
  }
  // Pass-1 grid.  On the matrix cores the matrices whose rows allow 16-byte
  // accesses take the first workgroups and the others the rest, so that each
  // part runs in an instantiation of the kernel compiled for its access width
  // only (the narrow-access path alone would raise the wide one's register
  // count); the vector path keeps the matrix order.
  for (int part = 0; part < (mfma ? 2 : 1); ++part) {
    for (size_t k = 0; k < p->mats.size(); ++k) {
      MatDesc& d = p->mats[k];
      if (mfma && (part == 0) != (d.vec == 4)) continue;
      d.wg_rows0 = wg_rows;
      for (int32_t t = 0; t < p->nrow_wg[k]; ++t) p->rows_map.push_back((int32_t)k);
      wg_rows += p->nrow_wg[k];
    }
    if (part == 0) p->hdr.wg_rows_v4 = mfma ? wg_rows : 0;
  }
  // orthonormalisation descriptors: P of compress, P and Q of the refresh
  const size_t nm = p->mats.size();
  p->orth.resize(3 * nm);
  int32_t wg_gramq = 0;
  for (size_t k = 0; k < nm; ++k) {
    const MatDesc& d = p->mats[k];
    OrthDesc o{};
    o.gram_off = d.gram_off;
    o.t_off = d.t_off;
    o.rows = d.m;
    o.ngb = (d.m + kGramRows - 1) / kGramRows;
    o.off = d.p_off;
    o.wg0 = d.wg_gram0;
    p->orth[k] = o;
    o.off = 0;
    o.wg0 = 0;
    p->orth[nm + k] = o;
    o.rows = d.n;
    o.ngb = (d.n + kGramRows - 1) / kGramRows;
    o.off = d.q_off;
    o.wg0 = wg_gramq;
    for (int32_t t = 0; t < o.ngb; ++t) p->gramq_map.push_back((int32_t)k);
    wg_gramq += o.ngb;
    p->orth[2 * nm + k] = o;
  }
  // the grouped refresh inside compress keeps its P in the refresh scratch
  // with the P buffer's layout
  rscr = std::max<int64_t>(rscr, (int64_t)p->p_elems);
  int32_t wg_pass = 0;
  for (size_t k = 0; k < p->pass.size(); ++k) {
    PassDesc& pd = p->pass[k];
    pd.wg0 = wg_pass;
    const int32_t nw = (int32_t)((pd.len + kPassChunk - 1) / kPassChunk);
    for (int32_t t = 0; t < nw; ++t) p->pass_map.push_back((int32_t)k);
    wg_pass += nw;
  }

  // Workspace layout: header and tables, then scratch.
  WsHeader& h = p->hdr;
  h.magic = kWsMagic;
  h.nmat = (int32_t)p->mats.size();
  h.npass = (int32_t)p->pass.size();
  h.rank = rank;
  h.flags = (int32_t)flags;
  h.wg_rows = wg_rows;
  h.wg_rec = wg_rec;
  h.wg_mtp = wg_mtp;
  h.wg_red = wg_red;
  h.wg_pass = wg_pass;
  h.wg_pred = wg_pred;
  h.wg_gram = wg_gram;
  h.wg_gramq = wg_gramq;
  h.rank_pad = (int32_t)rp;
  h.mfma = mfma ? 1 : 0;
  int64_t b = align_up(sizeof(WsHeader), 256);
  h.mat_off = b;
  b = align_up(b + (int64_t)sizeof(MatDesc) * h.nmat, 256);
  h.pass_off = b;
  b = align_up(b + (int64_t)sizeof(PassDesc) * h.npass, 256);
  h.rows_map_off = b;
  b = align_up(b + 4 * (int64_t)p->rows_map.size(), 256);
  h.rec_map_off = b;
  b = align_up(b + 4 * (int64_t)p->rec_map.size(), 256);
  h.mtp_map_off = b;
  b = align_up(b + 4 * (int64_t)p->mtp_map.size(), 256);
  h.red_map_off = b;
  b = align_up(b + 4 * (int64_t)p->red_map.size(), 256);
  h.pass_map_off = b;
  b = align_up(b + 4 * (int64_t)p->pass_map.size(), 256);
  h.pred_map_off = b;
  b = align_up(b + 4 * (int64_t)p->pred_map.size(), 256);
  h.gram_map_off = b;
  b = align_up(b + 4 * (int64_t)p->gram_map.size(), 256);
  h.gramq_map_off = b;
  b = align_up(b + 4 * (int64_t)p->gramq_map.size(), 256);
  h.orth_off = b;
  b = align_up(b + (int64_t)sizeof(OrthDesc) * (int64_t)p->orth.size(), 256);
  h.tables_bytes = b;
  h.part_base = b;
  b = align_up(b + 4 * part, 256);
  h.ppart_base = b;
  b = align_up(b + (mfma ? 8 : 4) * ppart, 256);  // fp64 partials on the matrix cores
  h.gram_base = b;
  b = align_up(b + 8 * gram, 256);
  h.refresh_base = b;
  b = align_up(b + 4 * rscr, 256);
  h.total_bytes = b;

  p->tables.assign((size_t)h.tables_bytes, 0);
  memcpy(p->tables.data(), &h, sizeof h);
  if (h.nmat) memcpy(p->tables.data() + h.mat_off, p->mats.data(), sizeof(MatDesc) * h.nmat);
  if (h.npass) memcpy(p->tables.data() + h.pass_off, p->pass.data(), sizeof(PassDesc) * h.npass);
  if (!p->rows_map.empty())
    memcpy(p->tables.data() + h.rows_map_off, p->rows_map.data(), 4 * p->rows_map.size());
  if (!p->rec_map.empty())
    memcpy(p->tables.data() + h.rec_map_off, p->rec_map.data(), 4 * p->rec_map.size());
  if (!p->mtp_map.empty())
    memcpy(p->tables.data() + h.mtp_map_off, p->mtp_map.data(), 4 * p->mtp_map.size());
  if (!p->red_map.empty())
    memcpy(p->tables.data() + h.red_map_off, p->red_map.data(), 4 * p->red_map.size());
  if (!p->pass_map.empty())
    memcpy(p->tables.data() + h.pass_map_off, p->pass_map.data(), 4 * p->pass_map.size());
  if (!p->pred_map.empty())
    memcpy(p->tables.data() + h.pred_map_off, p->pred_map.data(), 4 * p->pred_map.size());
  if (!p->gram_map.empty())
    memcpy(p->tables.data() + h.gram_map_off, p->gram_map.data(), 4 * p->gram_map.size());
  if (!p->gramq_map.empty())
    memcpy(p->tables.data() + h.gramq_map_off, p->gramq_map.data(), 4 * p->gramq_map.size());
  if (!p->orth.empty())
    memcpy(p->tables.data() + h.orth_off, p->orth.data(), sizeof(OrthDesc) * p->orth.size());

  *out = p;
  return PSGD_OK;
}

extern "C" psgd_status_t psgd_plan_get_info(psgd_plan_t p, psgd_plan_info_t* info) {
  clear_error();
  if (!p || !info) {
    set_error("psgd_plan_get_info: NULL argument");
    return PSGD_ERR_INVALID_ARG;
  }
  memset(info, 0, sizeof *info);
  info->ntensors = p->ntensors;
  info->ncompressed = (int32_t)p->mats.size();
  info->rank = p->rank;
  info->flags = p->flags;
  info->flat_elems = p->flat_elems;
  info->p_elems = p->p_elems;
  info->passthru_elems = p->pt_elems;
  info->p_buffer_elems = p->p_elems + p->pt_elems;
  info->q_elems = p->q_elems;
  info->payload_elems = p->payload;
  info->dense_elems = p->dense;
  info->workspace_bytes = (size_t)p->hdr.total_bytes;
  return PSGD_OK;
}

extern "C" psgd_status_t psgd_plan_tensor(psgd_plan_t p, int32_t t, int32_t* kind, int64_t* flat_off,
                                          int64_t* p_off, int64_t* q_off) {
  clear_error();
  if (!p) {
    set_error("psgd_plan_tensor: plan is NULL");
    return PSGD_ERR_INVALID_ARG;
  }
  if (t < 0 || t >= p->ntensors) {
    set_error("psgd_plan_tensor: tensor %d out of range [0, %d)", t, p->ntensors);
    return PSGD_ERR_INVALID_ARG;
  }
  if (kind) *kind = p->kind[t];
  if (flat_off) *flat_off = p->flat_off[t];
  if (p_off) *p_off = p->p_off[t];
  if (q_off) *q_off = p->q_off[t];
  return PSGD_OK;
}

extern "C" const char* psgd_last_error(void) { return g_err; }

extern "C" const char* psgd_version(void) { return "psgd-mi355x 0.1 (gfx950)"; }
