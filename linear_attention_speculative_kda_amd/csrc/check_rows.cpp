// Host-side check of the row metadata (kda_check_rows in include/kda.h):
// plain C++ on host arrays, no device code. The kernels range-check every
// index they read, so bad metadata cannot make them access memory out of
// bounds; this check finds the rows that break the method's preconditions
// (distinct slots per request, windows within the caller's bound, record
// rows in range and distinct) before a call, for debugging.

#include <stdint.h>

#include <vector>

#include "kda.h"

extern "C" {

kda_status kda_check_rows(const int32_t* cu_seqlens, int32_t num_rows, int32_t num_tokens,
                          const int32_t* state_indices, int32_t num_slots,
                          const int32_t* record_rows, int32_t rec_rows, int32_t max_seqlen,
                          int32_t* bad_row, int32_t* issue) {
  if (bad_row) *bad_row = -1;
  if (issue) *issue = KDA_ROW_OK;
  if (num_rows < 0 || num_tokens < 0 || num_slots < 0 || max_seqlen < 0) return KDA_ERR_SHAPE;
  if (num_rows == 0) return KDA_OK;
  if (!cu_seqlens || !state_indices) return KDA_ERR_NULL;
  std::vector<unsigned char> slot_used((size_t)num_slots, 0);
  std::vector<unsigned char> rec_used(rec_rows > 0 ? (size_t)rec_rows : 0, 0);
  auto fail = [&](int row, kda_row_issue what) {
    if (bad_row) *bad_row = row;
    if (issue) *issue = what;
    return KDA_ERR_METADATA;
  };
  for (int i = 0; i < num_rows; ++i) {
    const int slot = state_indices[i];
    if (slot <= 0) continue;   // a skipped row
    const long long bos = cu_seqlens[i], eos = cu_seqlens[i + 1];
    if (bos < 0 || eos < bos || eos > num_tokens) return fail(i, KDA_ROW_SPAN);
    if (max_seqlen > 0 && eos - bos > max_seqlen) return fail(i, KDA_ROW_WINDOW);
    if (slot >= num_slots) return fail(i, KDA_ROW_SLOT_RANGE);
    if (slot_used[slot]) return fail(i, KDA_ROW_SLOT_DUP);
    slot_used[slot] = 1;
    if (rec_rows >= 0) {
      const int r = record_rows ? record_rows[i] : i;
      if (r < -1 || r >= rec_rows) return fail(i, KDA_ROW_RECORD_RANGE);
      if (r >= 0) {
        if (rec_used[r]) return fail(i, KDA_ROW_RECORD_DUP);
        rec_used[r] = 1;
      }
    }
  }
  return KDA_OK;
}

}  // extern "C"
