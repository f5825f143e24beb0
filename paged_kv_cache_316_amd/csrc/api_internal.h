// Host-side pieces of the decode entry point shared by pa_decode and the
// allocation-free variant: the argument checks and the launch.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pa {

struct DecodeCall {
  void* out;
  const void* q;
  const pa_pool* pool;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  const int32_t* seq_lens;
  int32_t num_seqs, num_q_heads;
  float scale;
  int32_t num_workers;
};

// Every host-checkable argument of a decode call except the workspace; on
// success *need is the workspace it needs in bytes (0 when num_seqs == 0, a
// call with nothing to do). Records the message of a failure.
pa_status decode_check(const DecodeCall& c, const char* who, size_t* need);
// Queues the decode kernels of a call that passed decode_check; `workspace`
// is device memory of at least *need bytes, 16-byte aligned.
pa_status decode_launch(const DecodeCall& c, void* workspace, void* stream, const char* who);

}  // namespace pa
