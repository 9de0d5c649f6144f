// Host-side stand-ins for the kernel launchers of libragattn (the functions
// ra_internal.h declares), for building the C ABI layer (capi.cpp) without
// its kernels: under host sanitizers and on a machine with no GPU. Each
// launcher records what it was given and returns the status set with
// stub_set_status(). All access goes through one mutex, so the records can
// be read from any thread.
#pragma once

#include "ra_internal.h"

struct StubRecord {
  int attn_calls = 0, merge_calls = 0, mla_calls = 0, append_calls = 0;
  ra::AttnParams attn{};
  int attn_bf16 = -1, attn_head_dim = -1;
  ra::KvLayout attn_layout = ra::kContiguous;
  ra::MaskKind attn_mask = ra::kMaskCausal;
  ra::MergeParams merge{};
  int merge_bf16 = -1, merge_head_dim = -1;
  ra::MlaParams mla{};
  int mla_bf16 = -1;
  ra::AppendParams append{};
  int append_bf16 = -1, append_head_dim = -1;
  int waves_override = 0;
};

// Clears the records and makes every later launch return hipSuccess.
void stub_reset();
// Status the next launches return.
void stub_set_status(hipError_t e);
// A copy of the records.
StubRecord stub_record();
