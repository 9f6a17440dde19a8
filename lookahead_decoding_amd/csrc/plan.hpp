// Launch plans of the attention and LM-head calls, shared by the entry
// points and the workspace query so all three always agree.
#pragma once

#include "attn_plan.hpp"
#include "head_plan.hpp"

namespace lopa {

inline size_t workspace_bytes(const lopa_dims& d) {
  const size_t a = attn_workspace_bytes(d);
  const size_t h = lmhead_workspace_bytes(d);
  return a > h ? a : h;
}

}  // namespace lopa
