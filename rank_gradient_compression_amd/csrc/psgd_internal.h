// Host-side plan object and error reporting shared by the library's
// translation units.
#pragma once

#include <stdint.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/psgd.h"
#include "psgd_tables.h"

namespace psgd {

struct TimingState;  // defined with the launch code

void set_error(const char* fmt, ...);
void clear_error();

}  // namespace psgd

struct psgd_plan {
  uint64_t id = 0;  // unique per plan created in this process (never 0)
  int32_t ntensors = 0;
  int32_t rank = 0;
  uint32_t flags = 0;
  float beta = 0.f;

  // per tensor
  std::vector<int64_t> rows, cols, numel, flat_off, p_off, q_off;
  std::vector<int32_t> kind;

  // device tables (host copy) and their layout
  std::vector<psgd::MatDesc> mats;
  std::vector<int32_t> mat_tensor;  // tensor index of each compressed matrix
  std::vector<psgd::PassDesc> pass;
  std::vector<int32_t> rows_map, rec_map, mtp_map, red_map, pass_map, pred_map, gram_map, gramq_map;
  std::vector<int32_t> nrow_wg;  // pass-1 workgroups of each matrix
  std::vector<psgd::OrthDesc> orth;  // 3 * nmat
  psgd::WsHeader hdr{};
  std::vector<uint8_t> tables;  // hdr + all tables, as uploaded

  size_t flat_elems = 0, p_elems = 0, pt_elems = 0, q_elems = 0;
  size_t payload = 0, dense = 0;
  int32_t max_m = 0, max_n = 0;
  size_t flat_lds = 0;  // dynamic LDS of the residual pass (flat-tiled matrices), bytes

  std::mutex timing_mu;
  psgd::TimingState* timing = nullptr;
};
