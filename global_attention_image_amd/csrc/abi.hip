// Error reporting and event-based stage timing for the uhla C ABI.
#include <stdio.h>

#include <vector>

#include "uhla_internal.h"

namespace uhla {

static thread_local char g_detail[512] = "";

void set_detail(const char* msg) {
  snprintf(g_detail, sizeof(g_detail), "%s", msg ? msg : "");
}

void set_hip_detail(const char* where, hipError_t e) {
  snprintf(g_detail, sizeof(g_detail), "%s: %s (%d)", where, hipGetErrorString(e),
           static_cast<int>(e));
}

int fail_arg(const char* msg) {
  set_detail(msg);
  return UHLA_ERR_ARG;
}

int fail_unsupported(const char* msg) {
  set_detail(msg);
  return UHLA_ERR_UNSUPPORTED;
}

int check_launch(const char* where) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_hip_detail(where, e);
    return UHLA_ERR_HIP;
  }
  return UHLA_OK;
}

}  // namespace uhla

// A timer owns max_calls * UHLA_NUM_STAGES event pairs.  Call i records into slot i.
struct uhla_timer {
  int max_calls = 0;
  int calls = 0;
  std::vector<hipEvent_t> start, stop;  // [max_calls * UHLA_NUM_STAGES]
  std::vector<unsigned char> used;      // stage recorded in that call
};

namespace uhla {

int timer_begin(uhla_timer* t, int stage, hipStream_t s) {
  if (t->calls >= t->max_calls) return UHLA_OK;
  const int i = t->calls * UHLA_NUM_STAGES + stage;
  const hipError_t e = hipEventRecord(t->start[i], s);
  if (e != hipSuccess) return (set_hip_detail("hipEventRecord", e), UHLA_ERR_HIP);
  return UHLA_OK;
}

int timer_end(uhla_timer* t, int stage, hipStream_t s) {
  if (t->calls >= t->max_calls) return UHLA_OK;
  const int i = t->calls * UHLA_NUM_STAGES + stage;
  const hipError_t e = hipEventRecord(t->stop[i], s);
  if (e != hipSuccess) return (set_hip_detail("hipEventRecord", e), UHLA_ERR_HIP);
  t->used[i] = 1;
  return UHLA_OK;
}

int timer_commit(uhla_timer* t) {
  if (t->calls < t->max_calls) ++t->calls;
  return UHLA_OK;
}

}  // namespace uhla

extern "C" const char* uhla_strerror(int status) {
  switch (status) {
    case UHLA_OK: return "UHLA_OK";
    case UHLA_ERR_ARG: return "UHLA_ERR_ARG: invalid argument";
    case UHLA_ERR_UNSUPPORTED: return "UHLA_ERR_UNSUPPORTED: configuration not built";
    case UHLA_ERR_WORKSPACE: return "UHLA_ERR_WORKSPACE: workspace missing or too small";
    case UHLA_ERR_HIP: return "UHLA_ERR_HIP: HIP runtime error";
    default: return "unknown uhla status";
  }
}

extern "C" const char* uhla_last_error_detail(void) { return uhla::g_detail; }

extern "C" int uhla_timer_create(int max_calls, uhla_timer** out) {
  if (!out || max_calls < 1 || max_calls > 100000) return uhla::fail_arg("bad timer arguments");
  uhla_timer* t = new uhla_timer();
  t->max_calls = max_calls;
  const size_t n = static_cast<size_t>(max_calls) * UHLA_NUM_STAGES;
  t->start.assign(n, nullptr);
  t->stop.assign(n, nullptr);
  t->used.assign(n, 0);
  for (size_t i = 0; i < n; ++i) {
    hipError_t e = hipEventCreate(&t->start[i]);
    if (e == hipSuccess) e = hipEventCreate(&t->stop[i]);
    if (e != hipSuccess) {
      uhla::set_hip_detail("hipEventCreate", e);
      uhla_timer_destroy(t);
      return UHLA_ERR_HIP;
    }
  }
  *out = t;
  return UHLA_OK;
}

extern "C" int uhla_timer_destroy(uhla_timer* t) {
  if (!t) return UHLA_OK;
  // every event is destroyed even if one fails; the first failure is reported
  hipError_t first = hipSuccess;
  for (hipEvent_t e : t->start)
    if (e) {
      const hipError_t r = hipEventDestroy(e);
      if (first == hipSuccess) first = r;
    }
  for (hipEvent_t e : t->stop)
    if (e) {
      const hipError_t r = hipEventDestroy(e);
      if (first == hipSuccess) first = r;
    }
  delete t;
  if (first != hipSuccess) {
    uhla::set_hip_detail("hipEventDestroy", first);
    return UHLA_ERR_HIP;
  }
  return UHLA_OK;
}

extern "C" int uhla_timer_reset(uhla_timer* t) {
  if (!t) return uhla::fail_arg("null timer");
  t->calls = 0;
  for (auto& u : t->used) u = 0;
  return UHLA_OK;
}

extern "C" int uhla_timer_read(uhla_timer* t, double* stage_ms, int n_stages, int* calls) {
  if (!t || !stage_ms || n_stages < 0) return uhla::fail_arg("bad timer arguments");
  const int ns = n_stages < UHLA_NUM_STAGES ? n_stages : UHLA_NUM_STAGES;
  for (int s = 0; s < n_stages; ++s) stage_ms[s] = 0.0;
  for (int c = 0; c < t->calls; ++c)
    for (int s = 0; s < ns; ++s) {
      const int i = c * UHLA_NUM_STAGES + s;
      if (!t->used[i]) continue;
      hipError_t e = hipEventSynchronize(t->stop[i]);
      float ms = 0.0f;
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, t->start[i], t->stop[i]);
      if (e != hipSuccess) {
        uhla::set_hip_detail("hipEventElapsedTime", e);
        return UHLA_ERR_HIP;
      }
      stage_ms[s] += ms;
    }
  if (calls) *calls = t->calls;
  return UHLA_OK;
}
