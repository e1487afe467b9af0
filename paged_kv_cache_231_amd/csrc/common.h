// Internal declarations shared by the host sources of libpkv.
#pragma once

#include <cstddef>
#include <cstdint>

#include "pkv.h"

namespace pkv {

// Records `msg` (a string literal) as the calling thread's last error.
pkv_status fail(pkv_status code, const char *msg);
void clear_error();

// Offsets of the sections of a spec-v1 plan, derived from its header.
struct PlanLayout {
  uint32_t Q = 0, S = 0, W = 0, ps = 0, N = 0, R = 0, T = 0;
  size_t lens = 0, qseq = 0, qpos = 0, rows = 0, tiles = 0, table = 0, total = 0;
};

// Reads the header of `words`; checks magic, version and that the section
// sizes add up to `n_words`.
pkv_status read_layout(const uint32_t *words, size_t n_words, PlanLayout *out);

// Full check of a spec-v1 plan (header, every section, row/tile cover).
pkv_status validate_plan(const uint32_t *words, size_t n_words, PlanLayout *out);

// Write plan of an append on a valid plan: no two queries target one
// physical (page, slot).
pkv_status validate_writes(const uint32_t *words, const PlanLayout &L);

}  // namespace pkv
