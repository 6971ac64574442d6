// abi.hip - error state, version and the kernel-timer measurement hook.
#include <math.h>
#include <string.h>

#include <atomic>
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

// Device check: per device, 0 = not asked yet, 1 = gfx950, 2 = another
// architecture. Devices past the table are asked on every call.
constexpr int MAX_DEVICES = 64;
static std::atomic<int> g_dev_state[MAX_DEVICES];

int check_device(const std::string& fn) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(CSK_EUNSUPPORTED, fn + ": no HIP device is visible (a gfx950 device is required)");
  }
  int st = dev < MAX_DEVICES ? g_dev_state[dev].load(std::memory_order_relaxed) : 0;
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(CSK_EHIP, fn + ": hipGetDeviceProperties failed");
    }
    // gcnArchName reads "gfx950" or "gfx950:sramecc+:xnack-"
    const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                    (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':');
    st = ok ? 1 : 2;
    if (dev < MAX_DEVICES) g_dev_state[dev].store(st, std::memory_order_relaxed);
    if (!ok)
      return fail(CSK_EUNSUPPORTED,
                  fn + ": device " + std::to_string(dev) + " is " + prop.gcnArchName + ", not gfx950");
  }
  if (st != 1) return fail(CSK_EUNSUPPORTED, fn + ": device " + std::to_string(dev) + " is not gfx950");
  return CSK_OK;
}

// One armed timer for the process: the named kernel's next n launches get
// an event pair each. g_timer_cap is the only state a launch reads when no
// timer is armed (one relaxed atomic load); everything else is read and
// written under the lock.
static std::mutex g_timer_mu;
static char g_timer_name[64] = {0};
static hipEvent_t* g_ev_start = nullptr;
static hipEvent_t* g_ev_stop = nullptr;
static std::atomic<int> g_timer_cap{0};
static int g_timer_next = 0;
static int g_timer_pending = -1;

void timer_before(const char* kernel, hipStream_t s) {
  if (g_timer_cap.load(std::memory_order_relaxed) == 0) return;
  std::lock_guard<std::mutex> lk(g_timer_mu);
  const int cap = g_timer_cap.load(std::memory_order_relaxed);
  if (cap == 0 || g_timer_next >= cap || strcmp(kernel, g_timer_name) != 0) return;
  (void)hipEventRecord(g_ev_start[g_timer_next], s);
  g_timer_pending = g_timer_next;
}

void timer_after(const char* kernel, hipStream_t s) {
  if (g_timer_cap.load(std::memory_order_relaxed) == 0) return;
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

int csk_fp8kv_entry_bytes(int D, int d_rope) {
  if (D <= 0 || d_rope < 0 || d_rope > D || (d_rope & 1) || (D - d_rope) % 32) return 0;
  return csk::fp8kv_entry_bytes(D, d_rope);
}

int csk_kernel_timer_arm(const char* kernel, void** ev_start, void** ev_stop, int n) {
  if (!kernel || !ev_start || !ev_stop || n <= 0 || strlen(kernel) >= sizeof(csk::g_timer_name))
    return csk::fail(CSK_EINVAL, "csk_kernel_timer_arm: bad arguments");
  std::lock_guard<std::mutex> lk(csk::g_timer_mu);
  strcpy(csk::g_timer_name, kernel);
  csk::g_ev_start = reinterpret_cast<hipEvent_t*>(ev_start);
  csk::g_ev_stop = reinterpret_cast<hipEvent_t*>(ev_stop);
  csk::g_timer_next = 0;
  csk::g_timer_pending = -1;
  csk::g_timer_cap.store(n, std::memory_order_relaxed);
  return CSK_OK;
}

int csk_kernel_timer_count(void) {
  std::lock_guard<std::mutex> lk(csk::g_timer_mu);
  return csk::g_timer_next;
}

void csk_kernel_timer_disarm(void) {
  std::lock_guard<std::mutex> lk(csk::g_timer_mu);
  csk::g_timer_cap.store(0, std::memory_order_relaxed);
  csk::g_timer_pending = -1;
  csk::g_ev_start = csk::g_ev_stop = nullptr;
}

}  // extern "C"
