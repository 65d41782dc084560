// RAII event pair around one kernel launch (active only while profiling is enabled).
#pragma once

#include <hip/hip_runtime.h>

namespace rf {

class ProfileScope {
 public:
  ProfileScope(int id, hipStream_t s);
  ~ProfileScope();
  ProfileScope(const ProfileScope&) = delete;
  ProfileScope& operator=(const ProfileScope&) = delete;

 private:
  int id_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr, stop_ = nullptr;
};

}  // namespace rf
