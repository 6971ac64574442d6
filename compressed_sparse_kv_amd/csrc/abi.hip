// abi.hip - error state, version and the kernel-timer measurement hook.
#include <math.h>
#include <string.h>

#include <mutex>

#include "common.h"

namespace csk {

static thread_local std::string g_err;

void set_error(const std::string& msg) { g_err = msg; }
int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}
void clear_error() { g_err.clear(); }

void fill_rope_table(RopeTable* t, int d_rope, double base) {
  for (int j = 0; j < MAX_ROPE_PAIRS; ++j)
    t->theta[j] = (2 * j < d_rope) ? pow(base, -2.0 * (double)j / (double)d_rope) : 0.0;
}

// One armed timer for the process: the named kernel's next n launches get
// an event pair each.
static std::mutex g_timer_mu;
static char g_timer_name[64] = {0};
static hipEvent_t* g_ev_start = nullptr;
static hipEvent_t* g_ev_stop = nullptr;
static int g_timer_cap = 0;
static int g_timer_next = 0;
static int g_timer_pending = -1;

void timer_before(const char* kernel, hipStream_t s) {
  if (g_timer_cap == 0) return;
  std::lock_guard<std::mutex> lk(g_timer_mu);
  if (g_timer_cap == 0 || g_timer_next >= g_timer_cap || strcmp(kernel, g_timer_name) != 0) return;
  (void)hipEventRecord(g_ev_start[g_timer_next], s);
  g_timer_pending = g_timer_next;
}

void timer_after(const char* kernel, hipStream_t s) {
  if (g_timer_cap == 0) return;
  std::lock_guard<std::mutex> lk(g_timer_mu);
  if (g_timer_pending < 0 || strcmp(kernel, g_timer_name) != 0) return;
  (void)hipEventRecord(g_ev_stop[g_timer_pending], s);
  g_timer_pending = -1;
  ++g_timer_next;
}

}  // namespace csk

extern "C" {

const char* csk_last_error(void) { return csk::g_err.c_str(); }

int csk_abi_version(void) { return CSK_ABI_VERSION; }

int csk_kernel_timer_arm(const char* kernel, void** ev_start, void** ev_stop, int n) {
  if (!kernel || !ev_start || !ev_stop || n <= 0 || strlen(kernel) >= sizeof(csk::g_timer_name))
    return csk::fail(CSK_EINVAL, "csk_kernel_timer_arm: bad arguments");
  std::lock_guard<std::mutex> lk(csk::g_timer_mu);
  strcpy(csk::g_timer_name, kernel);
  csk::g_ev_start = reinterpret_cast<hipEvent_t*>(ev_start);
  csk::g_ev_stop = reinterpret_cast<hipEvent_t*>(ev_stop);
  csk::g_timer_next = 0;
  csk::g_timer_pending = -1;
  csk::g_timer_cap = n;
  return CSK_OK;
}

int csk_kernel_timer_count(void) { return csk::g_timer_next; }

void csk_kernel_timer_disarm(void) {
  std::lock_guard<std::mutex> lk(csk::g_timer_mu);
  csk::g_timer_cap = 0;
  csk::g_ev_start = csk::g_ev_stop = nullptr;
}

}  // extern "C"
